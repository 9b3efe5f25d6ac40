"""GPU parity of the MX GEMM against the oracle's plain definition: exactly
dequantized MX operands, float64 products and sums (block-scaled tensor-core
compute: "Nvidia добивается успеха с 4-битным форматом NVFP4", asector.ru,
section "NVFP4 и Blackwell"; MXFP8 in the backward pass: "Thinking Machines
ускорила обучение Inkling 2 Small 4-битными числами", iitak.ru, section "Как
это работает").  Both accumulation modes of nvfp4_mx_gemm are checked.

EXACT mode is held to the criterion of the NVFP4 GEMM: per output
    |gpu - oracle| <= 1e-5 * sum_k |a_k b_k|
plus half a BF16 unit of the reference for BF16 outputs.  Every product is
exact there (BF16 matrix cores on exactly rescaled elements) and the sums are
binary32, as for nvfp4_gemm.

NATIVE mode (the scaled matrix cores) is checked against the precision this
hardware gives the block dot products, which the OCP Microscaling definition
leaves to the implementation; it does not meet the criterion above for E4M3
and is not claimed to.  An E2M1 step (64 products of at most 4 significant
bits each) is summed exactly and the per-step results are added in binary32;
an E4M3 step is summed with about 13 significant bits relative to the step's
largest product (measured: error up to ~2^-12 of that product).  Hence, per
output,
    |gpu - oracle| <= 2^-11 * sum over K steps of max_k |a_k b_k|   (E4M3 only)
                      + max(1e-5, steps * 2^-24) * sum_k |a_k b_k|
plus half a BF16 unit for BF16 outputs.

Operands whose products are all multiples of one power of two, with few
significant bits, have exactly representable sums: there both formats and
both modes must match exactly."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from oracle import banded as OB
from parity_utils import bf16_tensor_to_bits, require_gpu

pytestmark = pytest.mark.gpu

ELEMS = [O.MX_FP8, O.MX_FP4]


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def up(nv, q):
    return nv.MXTensor(torch.from_numpy(np.ascontiguousarray(q.codes)).cuda(),
                       torch.from_numpy(np.ascontiguousarray(q.scales)).cuda(), q.rows, q.cols, q.elem)


def step_max_sum(A, B, mi, ni):
    """sum over 64-wide K steps of max |a_k b_k| for entries (mi, ni); A, B
    exact float64 dequantizations."""
    K = A.shape[1]
    out = np.zeros(len(mi))
    for s in range(0, len(mi), 4096):
        P = np.abs(A[mi[s:s + 4096]] * B[ni[s:s + 4096]])
        out[s:s + 4096] = P.reshape(P.shape[0], K // 64, 64).max(-1).sum(-1)
    return out


NATIVE, EXACT = 0, 1
ACCUMS = [NATIVE, EXACT]


def tolerance(elem, K, W_, smax, cref, bf16, accum=NATIVE):
    if accum == EXACT:
        tol = 1e-5 * W_
    else:
        tol = max(1e-5, (K // 64) * 2.0 ** -24) * W_
        if elem == O.MX_FP8:
            tol = tol + 2.0 ** -11 * smax
    if bf16:
        a = np.abs(cref)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        tol = tol + np.where(a > 0, 2.0 ** (e - 8), 0.0)
    return tol


def check(nv, qa, qb, bf16=False, entries=None, exact=False, what="", accum=NATIVE, out=None, workspace=None):
    C = nv.nvfp4_mx_gemm(up(nv, qa), up(nv, qb), out_dtype=torch.bfloat16 if bf16 else torch.float32,
                         accum=accum, out=out, workspace=workspace)
    torch.cuda.synchronize()
    C = C.contiguous()
    if bf16:
        G = W.bf16_bits_to_f32(bf16_tensor_to_bits(C)).astype(np.float64)
    else:
        G = C.cpu().numpy().astype(np.float64)
    M, N, K = qa.rows, qb.rows, qa.cols
    if entries is None:
        mi, ni = (a.ravel() for a in np.meshgrid(np.arange(M), np.arange(N), indexing="ij"))
        Cref, Wref = OB.mx_gemm(qa, qb)
        Cref, Wref = Cref.ravel(), Wref.ravel()
    else:
        mi, ni = entries
        Cref, Wref = OB.mx_gemm(qa, qb, entries=(mi, ni))
    got = G[mi, ni]
    if exact:
        ref = Cref.astype(np.float32).astype(np.float64) if not bf16 else Cref
        assert np.array_equal(got, ref), f"{what}: exact case differs at {np.argmax(got != ref)}"
        return
    A = O.mx_dequantize(qa, 2)
    B = O.mx_dequantize(qb, 2)
    smax = step_max_sum(A, B, mi, ni) if (qa.elem == O.MX_FP8 and accum == NATIVE) else 0.0
    tol = tolerance(qa.elem, K, Wref, smax, Cref, bf16, accum)
    err = np.abs(got - Cref)
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, (f"{what} accum={accum}: {bad.size} entries off, first ({mi[bad[0]]}, {ni[bad[0]]}) "
                           f"gpu={got[bad[0]]!r} ref={Cref[bad[0]]!r} tol={tol[bad[0]] if np.ndim(tol) else tol!r}")


def mxq(x, elem, seed=0, rnd=O.RNE):
    return OB.mx_quantize(np.ascontiguousarray(x, dtype=np.float32), O.F32, elem, rnd, seed=seed)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("shape", [(64, 64, 64), (300, 260, 512), (256, 512, 4096)])
def test_mx_gemm_exact_case(nv, elem, shape, accum):
    """Elements in {0, +-1/2, +-1, +-2} with every block maximum 2: equal
    block scales, products on one power-of-two grid, sums below 2^15 -- the
    GPU result must equal the exact product."""
    M, N, K = shape
    g = W.rng(M + N + K)
    v = np.array([0, .5, 1, 2, -.5, -1, -2], np.float32)
    xa, xb = g.choice(v, (M, K)), g.choice(v, (N, K))
    xa[:, ::32] = 2.0
    xb[:, ::32] = -2.0
    for bf16 in (False, True):
        check(nv, mxq(xa, elem), mxq(xb, elem), bf16=bf16, exact=not bf16, what=f"exact {shape} bf16={bf16}",
              accum=accum)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("kind", ["normal", "t3", "spiky"])
@pytest.mark.parametrize("shape", [(1, 1, 64), (33, 65, 128), (300, 260, 512), (512, 320, 1024), (300, 260, 2048),
                                   (264, 200, 3072)])
def test_mx_gemm_matches_oracle(nv, elem, kind, shape, accum):
    """Ragged M and N; K below and at the 1024 multiple that selects the
    full-line kernels (K = 1024, 2048, and 3072: an odd number of their
    16-step bodies) -- both native kernels and both exact-accumulation
    kernels (the full-line one, and the ring one that takes every K % 64 == 0
    with ragged steps padded) are covered on the same inputs."""
    M, N, K = shape
    seed = M * 3 + N * 5 + K
    if kind == "normal":
        xa, xb = W.normal((M, K), 1.0, seed=seed), W.normal((N, K), 1.0, seed=seed + 1)
    elif kind == "t3":
        xa, xb = W.student_t((M, K), 3.0, seed=seed), W.student_t((N, K), 3.0, seed=seed + 1)
    else:
        xa = W.with_spikes(W.normal((M, K), 1.0, seed=seed), 1e-3, 100.0, seed=seed + 2)
        xb = W.with_spikes(W.normal((N, K), 1.0, seed=seed + 1), 1e-3, 100.0, seed=seed + 3)
    qa, qb = mxq(xa, elem, seed, O.SR), mxq(xb, elem, seed + 1, O.SR)
    for bf16 in (False, True):
        check(nv, qa, qb, bf16=bf16, what=f"{kind} {shape} elem={elem} bf16={bf16}", accum=accum)


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_gemm_scale_spread(nv, elem):
    """Rows and K blocks scaled by 2^-40 .. 2^40 (block scales across most of
    the E8M0 range within one output's sum)."""
    M, N, K = 96, 160, 1024
    g = W.rng(77)
    xa = W.normal((M, K), 1.0, seed=78) * (np.float32(2.0) ** g.integers(-40, 40, (M, K // 32)).repeat(32, 1))
    xb = W.normal((N, K), 1.0, seed=79) * (np.float32(2.0) ** g.integers(-40, 40, (N, K // 32)).repeat(32, 1))
    check(nv, mxq(xa, elem), mxq(xb, elem), what="scale spread")


@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("shape", [(96, 160, 1024), (130, 70, 576)])
def test_mx_gemm_exact_mode_scale_spread(nv, elem, shape):
    """Exact mode with K blocks scaled by 2^-24 .. 2^24, so that with the
    data's own spread every row's block scales stay within the 2^54 of its
    largest in which the products are exact; zero blocks (E8M0 byte 0) among
    them, and elements over all E4M3 / E2M1 magnitudes."""
    M, N, K = shape
    g = W.rng(M + N + K)
    xa = W.student_t((M, K), 3.0, seed=M) * (np.float32(2.0) ** g.integers(-24, 25, (M, K // 32)).repeat(32, 1))
    xb = W.student_t((N, K), 3.0, seed=N) * (np.float32(2.0) ** g.integers(-24, 25, (N, K // 32)).repeat(32, 1))
    xa[:, 32:64] = 0.0
    xb[3, :] = 0.0
    for q in (mxq(xa, elem), mxq(xb, elem)):
        nz = q.scales.astype(np.int64)
        span = np.where(nz > 0, nz.max(1, keepdims=True) - nz, 0).max()
        assert span <= 54, span
    for bf16 in (False, True):
        check(nv, mxq(xa, elem), mxq(xb, elem), bf16=bf16, what=f"exact spread {shape}", accum=EXACT)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("elem", ELEMS)
def test_mx_gemm_zero_k_and_empty(nv, elem, accum):
    a = nv.MXTensor.empty(70, 0, elem)
    b = nv.MXTensor.empty(50, 0, elem)
    C = nv.nvfp4_mx_gemm(a, b, accum=accum)
    torch.cuda.synchronize()
    assert C.shape == (70, 50) and not C.any()
    e = nv.MXTensor.empty(0, 64, elem)
    C = nv.nvfp4_mx_gemm(e, nv.MXTensor.empty(8, 64, elem), accum=accum)
    torch.cuda.synchronize()
    assert C.shape == (0, 8)


@pytest.mark.parametrize("elem", ELEMS)
def test_mx_gemm_8192_sampled(nv, elem):
    """8192 x 8192 x 8192 (the benchmarked launch), operands quantized by the
    oracle from Student-t(3) BF16 data: 1024 random entries plus the corners
    of the output against the oracle's per-entry sums."""
    n = 8192
    xa = W.bf16_bits_to_f32(W.f32_to_bf16_bits(W.student_t((n, n), 3.0, seed=8200)))
    xb = W.bf16_bits_to_f32(W.f32_to_bf16_bits(W.student_t((n, n), 3.0, seed=8201)))
    qa, qb = mxq(xa, elem, 8202, O.SR), mxq(xb, elem, 8203, O.SR)
    g = W.rng(8204)
    mi = np.concatenate([g.integers(0, n, 1024), [0, 0, n - 1, n - 1, 255, 256]])
    ni = np.concatenate([g.integers(0, n, 1024), [0, n - 1, 0, n - 1, 256, 255]])
    for accum in ACCUMS:
        check(nv, qa, qb, entries=(mi, ni), what="8192 sampled", accum=accum)


@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("shape", [(512, 512, 1024), (300, 200, 1024), (300, 600, 4096)])
@pytest.mark.parametrize("bf16", [False, True])
def test_mx_gemm_strided_output(nv, elem, shape, accum, bf16):
    """C written into a column slice of a wider buffer (row pitch N + 96,
    first column 40): the output addressing of whole wave tiles comes from
    the row pitch.  At K = 4096 the 6 tiles' last round is split in four,
    and the parts' sum is written with that pitch too.  The
    slice matches the oracle, and every byte outside it keeps the buffer's
    fill."""
    M, N, K = shape
    qa = mxq(W.student_t((M, K), 3.0, seed=M + 31), elem)
    qb = mxq(W.student_t((N, K), 3.0, seed=N + 37), elem, seed=1)
    dt = torch.bfloat16 if bf16 else torch.float32
    big = torch.empty((M, N + 96), dtype=dt, device="cuda")
    big.view(torch.uint8).fill_(0xA5)
    check(nv, qa, qb, bf16=bf16, accum=accum, out=big[:, 40:40 + N], what=f"strided {shape}")
    es = big.element_size()
    raw = big.view(torch.uint8)
    assert bool((raw[:, :40 * es] == 0xA5).all()) and bool((raw[:, (40 + N) * es:] == 0xA5).all()), \
        "bytes outside the output slice were written"


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("accum", ACCUMS)
@pytest.mark.parametrize("elem", ELEMS)
@pytest.mark.parametrize("shape", [(768, 768, 4096), (700, 600, 5120)])
def test_mx_gemm_tail_split(nv, elem, shape, accum, bf16):
    """Both accumulation modes, both output types: a last round of tiles that
    would leave compute units idle, computed in parts along K (9 tiles: 4
    parts at K = 4096, 5 ragged at K = 5120) when the workspace is given; a
    BF16 output rounds the parts' binary32 sum once.  Split and unsplit
    (workspace=False) both against the oracle; the split result the same
    over two calls."""
    M, N, K = shape
    qa = mxq(W.student_t((M, K), 3.0, seed=M + 41), elem)
    qb = mxq(W.student_t((N, K), 3.0, seed=N + 43), elem, seed=1)
    A, B = up(nv, qa), up(nv, qb)
    dt = torch.bfloat16 if bf16 else torch.float32
    assert nv.nvfp4_mx_gemm_workspace_size(A, B, out_dtype=dt, accum=accum) > 0
    C1 = nv.nvfp4_mx_gemm(A, B, out_dtype=dt, accum=accum)
    C2 = nv.nvfp4_mx_gemm(A, B, out_dtype=dt, accum=accum)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16 if bf16 else torch.int32),
                       C2.view(torch.int16 if bf16 else torch.int32)), "split result differs between calls"
    check(nv, qa, qb, bf16=bf16, what=f"split {shape}", accum=accum)
    check(nv, qa, qb, bf16=bf16, what=f"unsplit {shape}", workspace=False, accum=accum)


@pytest.mark.parametrize("bf16", [False, True], ids=["f32", "bf16"])
@pytest.mark.parametrize("elem", ELEMS)
def test_mx_gemm_tail_split_uneven(nv, elem, bf16):
    """Exact accumulation, 16 x 22 tiles at K = 5120: on 256 compute units the
    last round is 96 tiles, split in two parts of unequal length (two and
    three units of 1024 K).  Split and unsplit against the oracle on sampled
    entries: 2048 anywhere and 2048 in rows 2816-4095 (the tile rows that
    hold the last round's tiles).  Where the device has another number of
    compute units the split differs or does not happen; the comparison
    still holds."""
    M, N, K = 4096, 5632, 5120
    qa = mxq(W.student_t((M, K), 3.0, seed=51), elem)
    qb = mxq(W.student_t((N, K), 3.0, seed=53), elem, seed=1)
    rng = np.random.default_rng(55)
    mi = np.concatenate([rng.integers(0, M, 2048), rng.integers(2816, M, 2048)])
    ni = rng.integers(0, N, 4096)
    check(nv, qa, qb, bf16=bf16, entries=(mi, ni), what="uneven split", accum=EXACT)
    check(nv, qa, qb, bf16=bf16, entries=(mi, ni), what="uneven unsplit", workspace=False, accum=EXACT)


@pytest.mark.parametrize("elem,accum,shape,parts", [
    (O.MX_FP4, NATIVE, (6144, 6144, 4096), 0),    # 64-tile last round, short K: not split
    (O.MX_FP4, NATIVE, (768, 768, 4096), 9 * 4),   # 9 lone tiles: 4 parts each
    (O.MX_FP4, NATIVE, (700, 600, 2048), 0),
    (O.MX_FP8, NATIVE, (700, 600, 2048), 9 * 2),
    (O.MX_FP8, EXACT, (6144, 6144, 4096), 64 * 4),
    (O.MX_FP4, NATIVE, (20480, 5120, 8192), 64 * 2),
])
def test_mx_split_plan_choices(nv, elem, accum, shape, parts):
    """The split plan's choices for the shapes its cost estimate was fitted
    on, as workspace sizes (parts x 256 x 256 binary32), on a 256-CU device:
    a native E2M1 last round of 64 tiles at K = 4096 or 2048 K is not split,
    lone tiles and the slower kernels are."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the plan depends on the compute unit count; these choices are for 256")
    M, N, K = shape
    e = nv.NVFP4_MX_E4M3 if elem == O.MX_FP8 else nv.NVFP4_MX_E2M1
    A, B = nv.MXTensor.empty(M, K, e), nv.MXTensor.empty(N, K, e)
    assert nv.nvfp4_mx_gemm_workspace_size(A, B, accum=accum) == parts * 256 * 256 * 4
