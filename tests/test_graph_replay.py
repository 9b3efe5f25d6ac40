"""HIP graph capture and two-stream use of the library's calls: a sequence covering every entry
point (quantize with its amax pass and with a given amax, the fused and 2D
layouts, dequantize, re-quantization, MX quantize/dequantize, both GEMMs and
the grouped GEMM with its SwiGLU epilogue and amax) is captured once and
replayed several times, with eager work that overwrites every output in
between; every replay must reproduce the eager results bit for bit.  The
library records only kernel launches (no memsets), which is what makes its
calls capturable."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity_utils import require_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def test_sequence_graph_replays_match_eager(nv):
    R, C = 512, 768
    x = to_device(W.f32_to_bf16_bits(W.student_t((R, C), 3.0, seed=31)))
    dev = "cuda"
    ws = torch.empty(nv.nvfp4_quantize_workspace_size(R, C) // 4 + 4, dtype=torch.float32, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    qr = nv.NVFP4Tensor.empty(R, C)
    qc = nv.NVFP4Tensor.empty(C, R)
    q2r, q2c = nv.NVFP4Tensor.empty(R, C), nv.NVFP4Tensor.empty(C, R)
    qb = nv.NVFP4Tensor.empty(R, C, nv.NVFP4_SCALE_2D)
    rq = nv.NVFP4Tensor.empty(C, R)
    y = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    mq = nv.MXTensor.empty(R, C, nv.NVFP4_MX_E4M3)
    my = torch.empty((R, C), dtype=torch.float32, device=dev)
    gc = torch.empty((R, R), dtype=torch.float32, device=dev)
    mc = torch.empty((R, R), dtype=torch.float32, device=dev)
    # grouped: 3 groups over the 512 rows, weights 3 x 64 x 768 (SwiGLU: F = 32)
    offs = torch.tensor([0, 100, 100, 512], dtype=torch.int64, device=dev)
    wq = nv.nvfp4_quantize(to_device(W.f32_to_bf16_bits(W.normal((192, C), 0.02, seed=32))),
                           layout=nv.NVFP4_BLK_2D)
    wstack = nv.NVFP4Tensor(wq.codes, wq.scales, wq.tensor_scale.repeat(3).contiguous(), 192, C,
                            nv.NVFP4_SCALE_2D)
    h = torch.empty((R, 32), dtype=torch.bfloat16, device=dev)
    hmax = torch.zeros(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def seq():
        nv.nvfp4_quantize(x, round=nv.NVFP4_SR, sr_seed=1, out=qr, workspace=ws, amax_out=amax)
        nv.nvfp4_quantize(x, layout=nv.NVFP4_COL_1D, round=nv.NVFP4_SR, sr_seed=2, out=qc, amax_in=amax)
        nv.nvfp4_quantize(x, layout=nv.NVFP4_ROW_COL_1D, round=nv.NVFP4_SR, sr_seed=3, out=(q2r, q2c),
                          amax_in=amax)
        nv.nvfp4_quantize(x, layout=nv.NVFP4_BLK_2D, out=qb, workspace=ws)
        nv.nvfp4_dequantize(qr, out=y)
        nv.nvfp4_requantize(qr, round=nv.NVFP4_SR, sr_seed=4, hadamard=True, hadamard_seed=5, out=rq,
                            workspace=ws)
        nv.nvfp4_mx_quantize(x, round=nv.NVFP4_SR, sr_seed=6, out=mq)
        nv.nvfp4_mx_dequantize(mq, out=my)
        nv.nvfp4_gemm(qr, q2r, out=gc)
        nv.nvfp4_mx_gemm(mq, mq, out=mc)
        nv.nvfp4_grouped_gemm(qr, offs, wstack, 3, epilogue=nv.NVFP4_EPI_SWIGLU, out=h, amax_out=hmax)

    outputs = [amax, qr.codes, qr.scales, qr.tensor_scale, qc.codes, qc.scales, q2r.codes, q2r.scales,
               q2c.codes, q2c.scales, qb.codes, qb.scales, qb.tensor_scale, y, rq.codes, rq.scales,
               rq.tensor_scale, mq.codes, mq.scales, my, gc, mc, h, hmax]

    seq()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work between replays: overwrite every output
        for t in outputs:
            t.view(torch.uint8).fill_(0x5A + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (t, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: output {k} differs"
    # and the eager results are the oracle's (one spot check: the row quantization)
    q = O.quantize(x.cpu().view(torch.int16).numpy().view(np.uint16), O.BF16, O.ROW_1D, O.SR, sr_seed=1)
    assert np.array_equal(ref[1].cpu().numpy(), q.codes) and np.array_equal(ref[2].cpu().numpy(), q.scales)


def test_split_gemms_graph_replays_match_eager(nv):
    """The GEMMs with a workspace: a last round of 9 tiles split along K runs
    as two or three launches (whole tiles, parts, their sum), for FP32 and
    BF16 outputs of nvfp4_gemm and nvfp4_mx_gemm (native E2M1, exact E4M3).
    Captured once, replayed with every output and the workspaces overwritten
    in between; each replay reproduces the eager outputs bit for bit."""
    M = N = 768
    K = 4096
    dev = "cuda"
    xa = to_device(W.f32_to_bf16_bits(W.student_t((M, K), 3.0, seed=61)))
    xb = to_device(W.f32_to_bf16_bits(W.student_t((N, K), 3.0, seed=62)))
    qa, qb = nv.nvfp4_quantize(xa), nv.nvfp4_quantize(xb)
    ma, mb = nv.nvfp4_mx_quantize(xa, elem=nv.NVFP4_MX_E2M1), nv.nvfp4_mx_quantize(xb, elem=nv.NVFP4_MX_E2M1)
    ea, eb = nv.nvfp4_mx_quantize(xa, elem=nv.NVFP4_MX_E4M3), nv.nvfp4_mx_quantize(xb, elem=nv.NVFP4_MX_E4M3)
    calls = []
    for dt in (torch.float32, torch.bfloat16):
        calls.append((nv.nvfp4_gemm, qa, qb, dt, {}, nv.nvfp4_gemm_workspace_size(qa, qb, out_dtype=dt)))
        calls.append((nv.nvfp4_mx_gemm, ma, mb, dt, {"accum": nv.NVFP4_MX_ACC_NATIVE},
                      nv.nvfp4_mx_gemm_workspace_size(ma, mb, out_dtype=dt, accum=nv.NVFP4_MX_ACC_NATIVE)))
        calls.append((nv.nvfp4_mx_gemm, ea, eb, dt, {"accum": nv.NVFP4_MX_ACC_EXACT},
                      nv.nvfp4_mx_gemm_workspace_size(ea, eb, out_dtype=dt, accum=nv.NVFP4_MX_ACC_EXACT)))
    assert all(c[5] > 0 for c in calls), [c[5] for c in calls]
    outs = [torch.empty((M, N), dtype=c[3], device=dev) for c in calls]
    wss = [torch.empty(c[5] // 4, dtype=torch.float32, device=dev) for c in calls]
    torch.cuda.synchronize()

    def seq():
        for (fn, a, b, dt, kw, _), o, w in zip(calls, outs, wss):
            fn(a, b, out_dtype=dt, out=o, workspace=w, **kw)

    seq()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs + wss:
            t.view(torch.uint8).fill_(0x3C + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: call {k} differs"


def test_two_streams_match_one_stream(nv):
    """The library keeps no state between calls: the same calls split over two
    streams (default priority), overlapping, give bit-identical outputs to
    the calls in order on one stream."""
    R, C = 1024, 1536
    dev = "cuda"
    x = to_device(W.f32_to_bf16_bits(W.student_t((R, C), 3.0, seed=41)))
    ws = torch.empty(nv.nvfp4_quantize_workspace_size(R, C) // 4 + 4, dtype=torch.float32, device=dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    qa, qb = nv.NVFP4Tensor.empty(R, C), nv.NVFP4Tensor.empty(C, R)
    q2r, q2c = nv.NVFP4Tensor.empty(R, C), nv.NVFP4Tensor.empty(C, R)
    qd = nv.NVFP4Tensor.empty(R, C, nv.NVFP4_SCALE_2D)
    rq = nv.NVFP4Tensor.empty(C, R)
    mq = nv.MXTensor.empty(R, C, nv.NVFP4_MX_E2M1)
    y = torch.empty((R, C), dtype=torch.bfloat16, device=dev)
    g = torch.empty((R, R), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    outputs = [amax, qa.codes, qa.scales, qb.codes, qb.scales, q2r.codes, q2r.scales, q2c.codes, q2c.scales,
               qd.codes, qd.scales, rq.codes, rq.scales, rq.tensor_scale, mq.codes, mq.scales, y, g]

    def run(split):
        main = torch.cuda.current_stream()
        nv.nvfp4_quantize(x, round=nv.NVFP4_SR, sr_seed=1, out=qa, workspace=ws, amax_out=amax)
        other = side if split else main
        other.wait_stream(main)
        with torch.cuda.stream(other):
            nv.nvfp4_quantize(x, layout=nv.NVFP4_COL_1D, round=nv.NVFP4_SR, sr_seed=2, out=qb, amax_in=amax)
            nv.nvfp4_requantize(qa, round=nv.NVFP4_SR, sr_seed=3, out=rq, workspace=ws)
            nv.nvfp4_mx_quantize(x, round=nv.NVFP4_SR, sr_seed=4, out=mq)
        nv.nvfp4_quantize(x, layout=nv.NVFP4_ROW_COL_1D, out=(q2r, q2c), amax_in=amax)
        nv.nvfp4_quantize(x, layout=nv.NVFP4_BLK_2D, out=qd, amax_in=amax)
        nv.nvfp4_dequantize(qa, out=y)
        nv.nvfp4_gemm(qa, q2r, out=g)
        main.wait_stream(other)

    run(False)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    for rep in range(3):
        for t in outputs:
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        run(True)
        torch.cuda.synchronize()
        for k, (t, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"rep {rep}: output {k} differs"


def test_stream_argument_keeps_workspace_on_that_stream(nv):
    """Calls given stream= (not torch's current stream) allocate their outputs
    and their amax workspace on that stream: work enqueued on the current
    stream right after the call returns, which allocates and overwrites
    memory, cannot receive the workspace the delayed kernels still read."""
    R, C = 512, 1024
    x = to_device(W.f32_to_bf16_bits(W.student_t((R, C), 3.0, seed=51)))
    xh = x.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = O.quantize(xh, O.BF16, O.ROW_1D, O.SR, sr_seed=7)
    ref_rq = O.requantize(ref, O.SR, sr_seed=8)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            torch.cuda._sleep(50_000_000)  # a bounded spin: the calls below start late
        q = nv.nvfp4_quantize(x, round=nv.NVFP4_SR, sr_seed=7, stream=side)
        rq = nv.nvfp4_requantize(q, round=nv.NVFP4_SR, sr_seed=8, stream=side)
        # the current stream now allocates and fills blocks of every small size
        junk = [torch.full((n,), 3.0e38, dtype=torch.float32, device="cuda") for n in (128, 256, 512, 1024)]
        torch.cuda.synchronize()
        del junk
        got = O.QTensor(q.codes.cpu().numpy(), q.scales.cpu().numpy(), float(q.tensor_scale[0].item()),
                        q.rows, q.cols, q.scale_mode)
        assert got.ts == ref.ts, f"rep {rep}: tensor scale {got.ts} != {ref.ts}"
        assert np.array_equal(got.codes, ref.codes) and np.array_equal(got.scales, ref.scales)
        assert float(rq.tensor_scale[0].item()) == ref_rq.ts
        assert np.array_equal(rq.codes.cpu().numpy(), ref_rq.codes)
        assert np.array_equal(rq.scales.cpu().numpy(), ref_rq.scales)
