"""GPU parity of the block-scaled GEMM and grouped GEMM against the oracle's
float64 dequantize-then-matmul: |gpu - oracle| <= 1e-5 * sum_k |a_k b_k| per
element (plus half a bf16 ulp for bf16 outputs)."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from oracle import banded as OB
from parity_utils import (assert_q_equal, bf16_tensor_to_bits, gemm_tol, q_to_device, q_to_host,
                          require_gpu, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def out_to_f64(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(bf16_tensor_to_bits(t)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def check(got, Cref, Wref, bf16_out, what):
    tol = gemm_tol(Cref, Wref, bf16_out)
    err = np.abs(got - Cref)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} entries out of tolerance, first {i.tolist()}: "
                             f"gpu={got[tuple(i)]!r} ref={Cref[tuple(i)]!r} tol={tol[tuple(i)]!r}")


def quant_host(x, layout, rnd=O.RNE, seed=0):
    return O.quantize(x, O.F32, layout, rnd, sr_seed=seed)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (32, 32, 64), (100, 70, 80), (130, 260, 1040),
                                   (300, 128, 4112), (257, 129, 48), (64, 256, 192), (96, 160, 320),
                                   (260, 300, 1024), (300, 260, 512), (33, 530, 1536)])
@pytest.mark.parametrize("bmode", [O.ROW_1D, O.BLK_2D])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_small(nv, M, N, K, bmode, out):
    if bmode == O.BLK_2D and N % 16:
        N = (N + 15) // 16 * 16
    a = W.with_spikes(W.student_t((M, K), 3.0, seed=M + K), 1e-3, 50.0, seed=1)
    b = W.normal((N, K), 0.02, seed=N + 3 * K)
    A, B = quant_host(a, O.ROW_1D), quant_host(b, bmode)
    C = nv.nvfp4_gemm(q_to_device(A, nv), q_to_device(B, nv),
                      out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    Cref, Wref = OB.gemm(A, B)
    check(out_to_f64(C), Cref, Wref, out == "bf16", f"gemm {M}x{N}x{K}")


def test_gemm_exact_unit_scales(nv):
    """Every block multiplier 1 and tensor scale 1: products are multiples of
    1/4 and sums stay below 2^24, so the FP32 result must be exact."""
    M, N, K = 160, 96, 512
    r = W.rng(5)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)

    def make(rows):
        x = grid[r.integers(0, 8, size=(rows, K))] * np.where(r.random((rows, K)) < 0.5, -1, 1)
        x = x.astype(np.float32)
        x[:, ::16] = 6.0
        return x

    A = O.quantize(make(M), O.F32, O.ROW_1D, amax_in=2688.0)
    B = O.quantize(make(N), O.F32, O.ROW_1D, amax_in=2688.0)
    C = nv.nvfp4_gemm(q_to_device(A, nv), q_to_device(B, nv))
    Cref, _ = OB.gemm(A, B)
    assert np.array_equal(out_to_f64(C), Cref)


def test_gemm_256_config(nv):
    """M = N = K = 256, A and B FP32 N(0,1) with 0.1% x50 outliers; A
    quantized along rows, B (K x N) along K (column blocks), RNE; FP32 out.
    The GPU's quantized operands equal the oracle's; the oracle's GEMM runs
    on its own quantization."""
    n = 256
    a = W.with_spikes(W.normal((n, n), 1.0, seed=1), 1e-3, 50.0, seed=2)
    b = W.with_spikes(W.normal((n, n), 1.0, seed=3), 1e-3, 50.0, seed=4)
    Ad = nv.nvfp4_quantize(to_device(a), layout=nv.NVFP4_ROW_1D)
    Bd = nv.nvfp4_quantize(to_device(b), layout=nv.NVFP4_COL_1D)   # B^T, N x K
    C = nv.nvfp4_gemm(Ad, Bd)
    Aref, Bref = O.quantize(a, O.F32, O.ROW_1D), O.quantize(b, O.F32, O.COL_1D)
    assert_q_equal(q_to_host(Ad), Aref, "A")
    assert_q_equal(q_to_host(Bd), Bref, "B")
    Cref, Wref = OB.gemm(Aref, Bref)
    check(out_to_f64(C), Cref, Wref, False, "gemm 256")


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (300, 224, 1024), (256, 384, 1024)])
@pytest.mark.parametrize("out", ["f32", "bf16", "swiglu"])
def test_gemm_strided_output(nv, M, N, K, out):
    """C written into a column slice of a wider buffer (row pitch = width +
    96, first column 40): whole wave tiles are written through offsets formed
    from the row pitch.  The slice matches the oracle (SwiGLU: its h), and
    every byte outside it keeps the buffer's fill."""
    a = W.student_t((M, K), 3.0, seed=M + 5)
    b = W.normal((N, K), 0.02, seed=N + 7)
    A, B = quant_host(a, O.ROW_1D), quant_host(b, O.BLK_2D)
    width = N // 2 if out == "swiglu" else N
    dt = torch.float32 if out == "f32" else torch.bfloat16
    big = torch.empty((M, width + 96), dtype=dt, device="cuda")
    big.view(torch.uint8).fill_(0xA5)
    C = big[:, 40:40 + width]
    if out == "swiglu":
        nv.nvfp4_gemm(q_to_device(A, nv), q_to_device(B, nv), out=C, epilogue=nv.NVFP4_EPI_SWIGLU)
    else:
        nv.nvfp4_gemm(q_to_device(A, nv), q_to_device(B, nv), out=C)
    got = out_to_f64(C.contiguous())
    Cref, Wref = OB.gemm(A, B)
    if out == "swiglu":
        F = width
        G_, U_ = Cref[:, :F], Cref[:, F:]
        err = np.abs(got - O.swiglu(G_, U_))
        tol = _swiglu_tol(G_, U_, Wref[:, :F], Wref[:, F:])
        assert (err <= tol).all(), f"strided swiglu: {np.sum(err > tol)} entries out of tolerance"
    else:
        check(got, Cref, Wref, out == "bf16", f"strided gemm {M}x{N}x{K}")
    es = big.element_size()
    raw = big.view(torch.uint8)
    assert bool((raw[:, :40 * es] == 0xA5).all()) and bool((raw[:, (40 + width) * es:] == 0xA5).all()), \
        "bytes outside the output slice were written"


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(768, 768, 4096), (700, 608, 2048), (300, 272, 1024)])
def test_gemm_tail_split(nv, M, N, K, out):
    """A last round of tiles that would leave compute units idle, computed in
    parts along K (FP32 and BF16 outputs, workspace given): against the oracle, the
    same over two calls, and the unsplit call (workspace=False) against the
    oracle too.  9 tiles at K = 4096 take 8 parts each; 9 ragged tiles at
    K = 2048, 4; 4 ragged tiles at K = 1024, 2."""
    a = W.student_t((M, K), 3.0, seed=M + 11)
    b = W.normal((N, K), 0.02, seed=N + 13)
    A, B = quant_host(a, O.ROW_1D), quant_host(b, O.BLK_2D)
    Ad, Bd = q_to_device(A, nv), q_to_device(B, nv)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    assert nv.nvfp4_gemm_workspace_size(Ad, Bd, out_dtype=dt) > 0
    C1 = nv.nvfp4_gemm(Ad, Bd, out_dtype=dt)
    C2 = nv.nvfp4_gemm(Ad, Bd, out_dtype=dt)
    C0 = nv.nvfp4_gemm(Ad, Bd, out_dtype=dt, workspace=False)
    Cref, Wref = OB.gemm(A, B)
    check(out_to_f64(C1), Cref, Wref, out == "bf16", f"split gemm {M}x{N}x{K}")
    check(out_to_f64(C0), Cref, Wref, out == "bf16", f"unsplit gemm {M}x{N}x{K}")
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16)), "split result differs between calls"


# -------------------------------------------------- full-size sampled checks
# At full size the oracle quantizes only the operand rows a sampled output
# needs, with the whole tensor's amax (rows of a row-blocked tensor and
# 16-row bands of a 2D-blocked one are independent given A_t; a column of a
# column-blocked tensor carries its own random-draw index base).  The GPU's
# quantized rows are checked equal to those, and the oracle's GEMM runs on
# the oracle's rows only.
def _oracle_rows(x, rows, amax):
    """Oracle nearest-even row-block quantization of rows `rows` of BF16 x."""
    return O.quantize(np.ascontiguousarray(x[np.asarray(rows)]), O.BF16, O.ROW_1D, amax_in=amax)


def _oracle_bands(x, rows, amax):
    """Oracle 16x16-block quantization of the 16-row bands holding `rows`;
    returns the stacked bands, their indices and each row's local index."""
    rows = np.asarray(rows)
    bands = np.unique(rows // 16)
    sub = np.concatenate([x[16 * b:16 * b + 16] for b in bands])
    q = O.quantize(sub, O.BF16, O.BLK_2D, amax_in=amax)
    return q, bands, np.searchsorted(bands, rows // 16) * 16 + rows % 16


def _oracle_cols(x, cols, amax, seed, hseed):
    """Oracle column-block quantization (Hadamard along the column, SR) of
    columns `cols` of BF16 x: rows of the transposed operand, each with the
    random-draw indices of its place in the whole output."""
    rows = x.shape[0]
    qs = [O.quantize(np.ascontiguousarray(x[:, c:c + 1]), O.BF16, O.COL_1D, O.SR, sr_seed=seed,
                     hadamard=True, hadamard_seed=hseed, amax_in=amax, index_base=int(c) * rows)
          for c in cols]
    return O.QTensor(np.concatenate([q.codes for q in qs]), np.concatenate([q.scales for q in qs]),
                     qs[0].ts, len(qs), rows, O.SCALE_1D)


def _assert_gpu_rows(qd, rows, ref, what, ts_index=0):
    """Rows `rows` of the device tensor qd (1D scales) equal the oracle's."""
    idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()
    got = O.QTensor(qd.codes.index_select(0, idx).cpu().numpy(), qd.scales.index_select(0, idx).cpu().numpy(),
                    float(qd.tensor_scale[ts_index].item()), len(rows), qd.cols, O.SCALE_1D)
    assert_q_equal(got, ref, what)


def _assert_gpu_bands(qd, bands, ref, what, row0=0, ts_index=0):
    """16-row bands `bands` (from row row0) of the 2D-scaled device tensor qd
    equal the oracle's stacked bands."""
    b = np.asarray(bands, dtype=np.int64)
    rows = (row0 + 16 * b[:, None] + np.arange(16)[None, :]).reshape(-1)
    codes = qd.codes.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
    scales = qd.scales.index_select(0, torch.from_numpy(row0 // 16 + b).cuda()).cpu().numpy()
    got = O.QTensor(codes, scales, float(qd.tensor_scale[ts_index].item()), rows.size, qd.cols, O.SCALE_2D)
    assert_q_equal(got, ref, what)


def _sample_entries(M, N, n, seed):
    r = W.rng(seed)
    mi = np.concatenate([r.integers(0, M, n), np.arange(8), M - 1 - np.arange(8)])
    ni = np.concatenate([r.integers(0, N, n), np.arange(8), N - 1 - np.arange(8)])
    return mi, ni


def test_forward_8192x20480x5120_sampled(nv):
    """Y = X W^T: X 8192 x 5120 Student-t(3) row blocks, W 20480 x 5120
    N(0, 0.02) 16x16 blocks, BF16 output; sampled entries."""
    x = W.f32_to_bf16_bits(W.student_t((8192, 5120), 3.0, seed=4000))
    w = W.f32_to_bf16_bits(W.normal((20480, 5120), 0.02, seed=4001))
    Xq = nv.nvfp4_quantize(to_device(x), layout=nv.NVFP4_ROW_1D)
    Wq = nv.nvfp4_quantize(to_device(w), layout=nv.NVFP4_BLK_2D)
    Y = nv.nvfp4_gemm(Xq, Wq, out_dtype=torch.bfloat16)
    mi, ni = _sample_entries(8192, 20480, 1024, 4002)
    ru, ml = np.unique(mi, return_inverse=True)
    Aq = _oracle_rows(x, ru, O.amax(x, O.BF16, O.ROW_1D))
    Bq, bands, nl = _oracle_bands(w, ni, O.amax(w, O.BF16, O.BLK_2D))
    _assert_gpu_rows(Xq, ru, Aq, "X rows")
    _assert_gpu_bands(Wq, bands, Bq, "W bands")
    Cref, Wref = OB.gemm(Aq, Bq, entries=(ml, nl))
    got = out_to_f64(Y)[mi, ni]
    check(got, Cref, Wref, True, "forward sampled")


def test_wgrad_20480x5120x8192_sampled(nv):
    """dW = dY^T X with K = 8192 tokens: both operands Hadamard-transformed
    along tokens with one shared sign seed, column blocks, SR; FP32 out."""
    dy = W.f32_to_bf16_bits(W.with_spikes(W.normal((8192, 20480), 1.0, seed=5000), 1e-4, 100.0, seed=5001))
    x = W.f32_to_bf16_bits(W.with_spikes(W.normal((8192, 5120), 1.0, seed=5002), 1e-4, 100.0, seed=5003))
    kw = dict(layout=nv.NVFP4_COL_1D, round=nv.NVFP4_SR, hadamard=True, hadamard_seed=5200)
    dYq = nv.nvfp4_quantize(to_device(dy), sr_seed=5100, **kw)
    Xq = nv.nvfp4_quantize(to_device(x), sr_seed=5101, **kw)
    dW = nv.nvfp4_gemm(dYq, Xq, out_dtype=torch.float32)
    mi, ni = _sample_entries(20480, 5120, 1024, 5003)
    mu, ml = np.unique(mi, return_inverse=True)
    nu, nl = np.unique(ni, return_inverse=True)
    Aq = _oracle_cols(dy, mu, O.amax(dy, O.BF16, O.COL_1D, hadamard=True, hadamard_seed=5200), 5100, 5200)
    Bq = _oracle_cols(x, nu, O.amax(x, O.BF16, O.COL_1D, hadamard=True, hadamard_seed=5200), 5101, 5200)
    _assert_gpu_rows(dYq, mu, Aq, "dY^T rows")
    _assert_gpu_rows(Xq, nu, Bq, "X^T rows")
    Cref, Wref = OB.gemm(Aq, Bq, entries=(ml, nl))
    check(out_to_f64(dW)[mi, ni], Cref, Wref, False, "wgrad sampled")


# ---------------------------------------------------------------- grouped
def _grouped_inputs(counts, N, K, seed, bmode=O.BLK_2D):
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    a = W.student_t((int(offs[-1]), K), 3.0, seed=seed)
    A = quant_host(a, O.ROW_1D)
    Bs = [quant_host(W.normal((N, K), 0.02, seed=seed + 1 + g), bmode) for g in range(len(counts))]
    return offs, A, Bs


def _stack_device(Bs, nv):
    codes = np.concatenate([b.codes for b in Bs])
    scales = np.concatenate([b.scales for b in Bs])
    ts = torch.tensor([b.ts for b in Bs], dtype=torch.float32, device="cuda")
    return nv.NVFP4Tensor(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), ts,
                          sum(b.rows for b in Bs), Bs[0].cols, Bs[0].scale_mode)


@pytest.mark.parametrize("counts", [[5, 0, 130, 64], [1], [0, 0, 300], [128, 128, 1, 255, 17]])
@pytest.mark.parametrize("bmode", [O.ROW_1D, O.BLK_2D])
def test_grouped_gemm_small(nv, counts, bmode):
    N, K = 96, 208
    offs, A, Bs = _grouped_inputs(counts, N, K, seed=sum(counts) + 7, bmode=bmode)
    C = nv.nvfp4_grouped_gemm(q_to_device(A, nv), torch.from_numpy(offs).cuda(), _stack_device(Bs, nv),
                              len(counts), out_dtype=torch.float32)
    Cref, Wref = O.grouped_gemm(A, offs, Bs)
    check(out_to_f64(C), Cref, Wref, False, f"grouped {counts}")


@pytest.mark.parametrize("counts", [[5, 0, 130, 64], [128, 128, 1, 255, 17]])
@pytest.mark.parametrize("bmode", [O.ROW_1D, O.BLK_2D])
def test_grouped_gemm_full_line_path(nv, counts, bmode):
    """K = 512: the full-line kernel (whole 128-byte code lines per row),
    ragged and empty groups, both scale layouts of the weights."""
    N, K = 96, 512
    offs, A, Bs = _grouped_inputs(counts, N, K, seed=sum(counts) + 11, bmode=bmode)
    C = nv.nvfp4_grouped_gemm(q_to_device(A, nv), torch.from_numpy(offs).cuda(), _stack_device(Bs, nv),
                              len(counts), out_dtype=torch.bfloat16)
    Cref, Wref = O.grouped_gemm(A, offs, Bs)
    check(out_to_f64(C), Cref, Wref, True, f"grouped full-line {counts}")


def _swiglu_tol(G_, U_, Wg, Wu):
    from scipy.special import expit
    s = expit(G_)
    dh_dg = np.abs(s * (1.0 + G_ * (1.0 - s)) * U_)
    dh_du = np.abs(G_ * s)
    h = np.abs(G_ * s * U_)
    # one BF16 rounding: half a spacing, at least the subnormal spacing 2^-133
    e = np.maximum(np.floor(np.log2(np.where(h > 0, h, 1.0))), -126.0)
    ulp = np.where(h > 0, 2.0 ** (e - 7), 2.0 ** -133)
    return dh_dg * 1e-5 * Wg + dh_du * 1e-5 * Wu + 1e-6 * h + ulp


def check_swiglu(nv, counts, F, K, seed):
    offs, A, Bs = _grouped_inputs(counts, 2 * F, K, seed)
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    H = nv.nvfp4_grouped_gemm(q_to_device(A, nv), torch.from_numpy(offs).cuda(), _stack_device(Bs, nv),
                              len(counts), epilogue=nv.NVFP4_EPI_SWIGLU, amax_out=amax)
    got = out_to_f64(H)
    Cref, Wref = O.grouped_gemm(A, offs, Bs)
    G_, U_ = Cref[:, :F], Cref[:, F:]
    href = O.swiglu(G_, U_)
    tol = _swiglu_tol(G_, U_, Wref[:, :F], Wref[:, F:])
    err = np.abs(got - href)
    assert (err <= tol).all(), f"swiglu: {np.sum(err > tol)} entries out of tolerance"
    assert amax.item() == np.abs(got).max()
    return H, amax, href


def test_grouped_swiglu_small(nv):
    check_swiglu(nv, [70, 0, 129, 33], F=80, K=160, seed=21)


def test_grouped_swiglu_full_line_path(nv):
    check_swiglu(nv, [70, 0, 129, 33], F=80, K=1024, seed=22)


@pytest.mark.parametrize("M,F,K", [(70, 80, 160), (257, 48, 192), (300, 144, 1024)])
@pytest.mark.parametrize("bmode", [O.ROW_1D, O.BLK_2D])
def test_gemm_swiglu_epilogue(nv, M, F, K, bmode):
    """The plain GEMM's SwiGLU epilogue (B = [gate; up], 2F rows): each of
    the three kernels (K % 64 != 0, K % 64 == 0, K % 512 == 0) against the
    oracle's SwiGLU of its own GEMM, within the GEMM bound carried through
    h = g sigmoid(g) u."""
    a = W.with_spikes(W.student_t((M, K), 3.0, seed=M + F), 1e-3, 50.0, seed=2)
    A = quant_host(a, O.ROW_1D)
    B = quant_host(W.normal((2 * F, K), 0.02, seed=K + F), bmode)
    H = nv.nvfp4_gemm(q_to_device(A, nv), q_to_device(B, nv), out_dtype=torch.bfloat16,
                      epilogue=nv.NVFP4_EPI_SWIGLU)
    assert tuple(H.shape) == (M, F)
    Cref, Wref = OB.gemm(A, B)
    G_, U_ = Cref[:, :F], Cref[:, F:]
    err = np.abs(out_to_f64(H) - O.swiglu(G_, U_))
    tol = _swiglu_tol(G_, U_, Wref[:, :F], Wref[:, F:])
    assert (err <= tol).all(), f"swiglu gemm: {np.sum(err > tol)} entries out of tolerance"


def test_swiglu_then_quantize_is_oracle_exact(nv):
    """The quantize step after the SwiGLU epilogue: the GPU quantizes its BF16
    H with the amax the epilogue produced; the oracle quantizes its own H
    (its float64 SwiGLU rounded to BF16).  Where the two H rows are
    bit-identical the codes and scale bytes must be too (the exp of the
    epilogue and of the oracle may differ in the last bit, which can move a
    BF16 rounding; such rows are left out, and most rows must remain)."""
    H, amax, href = check_swiglu(nv, [64, 100], F=64, K=128, seed=31)
    q = q_to_host(nv.nvfp4_quantize(H, layout=nv.NVFP4_ROW_1D, amax_in=amax))
    hb = bf16_tensor_to_bits(H)
    hr = W.f32_to_bf16_bits(href.astype(np.float32))
    ref = O.quantize(hr, O.BF16, O.ROW_1D)
    assert q.ts == ref.ts, "tensor scale (the largest |H| differs)"
    same = np.all(hb == hr, axis=1)
    assert same.mean() >= 0.5, f"only {same.sum()} of {same.size} H rows are bit-identical"
    assert np.array_equal(q.codes[same], ref.codes[same]) and np.array_equal(q.scales[same], ref.scales[same])


def test_moe_expert_forward_sampled(nv):
    """32 experts, hidden 7168, FFN 2048, 16384 tokens top-4 with Zipf(1.1)
    counts.  Up-projection with SwiGLU: the GPU path end to end (GPU
    quantization of X and W1), its quantized rows checked equal to the
    oracle's and sampled rows of H against the oracle's SwiGLU of its own
    GEMM.  Down-projection at the same shape: an oracle-quantized synthetic
    SwiGLU output [65536 x 2048] times GPU-quantized W2 (its bands checked
    equal to the oracle's), sampled rows against the oracle."""
    E, Hd, F, T = 32, 7168, 2048, 16384
    counts = W.zipf_expert_counts(E, T, 4, 1.1)
    offs, token = W.moe_routing(counts, T)
    x = W.f32_to_bf16_bits(W.student_t((T, Hd), 3.0, seed=6000))
    Xq = nv.nvfp4_quantize(to_device(x), layout=nv.NVFP4_ROW_1D)
    idx = torch.from_numpy(token).cuda()
    Aperm = nv.NVFP4Tensor(Xq.codes.index_select(0, idx), Xq.scales.index_select(0, idx),
                           Xq.tensor_scale, int(offs[-1]), Hd, nv.NVFP4_SCALE_1D)
    w1 = [W.f32_to_bf16_bits(W.normal((2 * F, Hd), 0.02, seed=6100 + e)) for e in range(E)]
    W1 = nv.NVFP4Tensor.empty(E * 2 * F, Hd, nv.NVFP4_SCALE_2D, n_scales=E)
    for e in range(E):
        q = nv.nvfp4_quantize(to_device(w1[e]), layout=nv.NVFP4_BLK_2D)
        W1.codes[e * 2 * F:(e + 1) * 2 * F].copy_(q.codes)
        W1.scales[e * 2 * F // 16:(e + 1) * 2 * F // 16].copy_(q.scales)
        W1.tensor_scale[e:e + 1].copy_(q.tensor_scale)
    offs_d = torch.from_numpy(offs).cuda()
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    H = nv.nvfp4_grouped_gemm(Aperm, offs_d, W1, E, epilogue=nv.NVFP4_EPI_SWIGLU, amax_out=amax)
    # sampled rows: first/last rows of a big, a middle and the smallest group
    ax = O.amax(x, O.BF16, O.ROW_1D)
    Hh = out_to_f64(H)
    for g_ in (0, 15, 31):
        r0, r1 = int(offs[g_]), int(offs[g_ + 1])
        rows = np.array([r0, r0 + 1, (r0 + r1) // 2, r1 - 1])
        Aq = _oracle_rows(x, token[rows], ax)
        _assert_gpu_rows(Aperm, rows, Aq, f"X rows of group {g_}")
        cols = np.arange(0, F, 37)
        Bq, bands, local = _oracle_bands(w1[g_], np.concatenate([cols, cols + F]),
                                         O.amax(w1[g_], O.BF16, O.BLK_2D))
        _assert_gpu_bands(W1, bands, Bq, f"W1 bands of expert {g_}", row0=g_ * 2 * F, ts_index=g_)
        mi = np.repeat(np.arange(rows.size), cols.size)
        gl, ul = np.tile(local[:cols.size], rows.size), np.tile(local[cols.size:], rows.size)
        Cg, Wg = OB.gemm(Aq, Bq, entries=(mi, gl))
        Cu, Wu = OB.gemm(Aq, Bq, entries=(mi, ul))
        href = O.swiglu(Cg, Cu)
        tol = _swiglu_tol(Cg, Cu, Wg, Wu)
        got = Hh[np.repeat(rows, cols.size), np.tile(cols, rows.size)]
        assert (np.abs(got - href) <= tol).all(), f"group {g_}"
    del H, Aperm, W1, Xq
    torch.cuda.empty_cache()
    # down projection: oracle-quantized SwiGLU-shaped input, GPU-quantized W2
    h = W.f32_to_bf16_bits(W.student_t((int(offs[-1]), F), 3.0, seed=6300) * np.float32(0.05))
    Hq = O.quantize(h, O.BF16, O.ROW_1D)
    W2 = nv.NVFP4Tensor.empty(E * Hd, F, nv.NVFP4_SCALE_2D, n_scales=E)
    w2 = {}
    for e in range(E):
        w2e = W.f32_to_bf16_bits(W.normal((Hd, F), 0.02, seed=6200 + e))
        if e in (0, 7, 31):
            w2[e] = w2e
        q = nv.nvfp4_quantize(to_device(w2e), layout=nv.NVFP4_BLK_2D)
        W2.codes[e * Hd:(e + 1) * Hd].copy_(q.codes)
        W2.scales[e * Hd // 16:(e + 1) * Hd // 16].copy_(q.scales)
        W2.tensor_scale[e:e + 1].copy_(q.tensor_scale)
    Y = nv.nvfp4_grouped_gemm(q_to_device(Hq, nv), offs_d, W2, E, out_dtype=torch.bfloat16)
    Yh = out_to_f64(Y)
    for g_ in (0, 7, 31):
        r0, r1 = int(offs[g_]), int(offs[g_ + 1])
        rows = np.array([r0, (r0 + r1) // 2, r1 - 1])
        cols = np.arange(3, Hd, 101)
        Bq, bands, local = _oracle_bands(w2[g_], cols, O.amax(w2[g_], O.BF16, O.BLK_2D))
        _assert_gpu_bands(W2, bands, Bq, f"W2 bands of expert {g_}", row0=g_ * Hd, ts_index=g_)
        mi = np.repeat(rows, cols.size)
        Cref, Wref = OB.gemm(Hq, Bq, entries=(mi, np.tile(local, rows.size)))
        check(Yh[mi, np.tile(cols, rows.size)], Cref, Wref, True, f"down group {g_}")
