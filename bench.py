"""Benchmark of the NVFP4 hot path on one MI355X.

Headline workload (one "step"): an 8192 x 8192 BF16 activation tensor drawn
from Student-t(3) is quantized to NVFP4 along rows and along columns
(transpose re-quantization), each with round-to-nearest-even and with
stochastic rounding, in separate calls and in the fused row+column call; the
first call computes the tensor amax and publishes it (amax_out), the other
five reuse it (amax_in), as a pipeline quantizing one tensor several ways
would; the row and column results are then dequantized back to BF16.  The
step is timed as HIP graph replays (one graph per input buffer, captured from
the same calls; --no-graph times eager launches; both are reported).
`value` is the algorithmic bytes of the step (input read once + codes +
scales per quantize call; codes + scales + output per dequantize call; the
amax pass is not credited) divided by the step time, in GB/s.  Inputs rotate over 4 device buffers (512 MiB) so that
consecutive steps do not hit in the 256 MB Infinity Cache.

Also reported, on the same JSON line:
  roofline     -- the dominant kernel of the step, timed alone with HIP events
                  on the launch stream, against the 8 TB/s HBM peak (per-kernel
                  figures are the median over interleaved rounds of back-to-back
                  launches: the stochastic-rounding kernels' clocks move by up to
                  ~15% between bursts; every round's figure is on the line);
  cpu_baseline -- the CPU oracle on a bounded sample of the same step;
  kernels      -- each step kernel timed alone, the 16x16-block, dequantize,
                  re-quantization and amax kernels, and (with the GEMMs) the
                  8192 x 20480 gradient's Hadamard + column-block + SR
                  quantization, amax given and computed;
  gemm         -- the block-scaled GEMMs: the 256^3 case, forward 8192x20480x5120 (BF16 out),
                  weight-gradient 20480x5120x8192 (FP32 out, Hadamard + column
                  blocks + SR operands) and the 32-expert MoE forward
                  (up-projection with SwiGLU, quantize, down-projection), in
                  TFLOP/s against the FP16 MFMA peak they run on and the FP4
                  peak;
  mx           -- the MX formats: MXFP8 / MXFP4 quantize and dequantize of the
                  step's tensor, the 8.25-bit expert-output codec (MXFP8 row
                  encode of a 65536 x 7168 BF16 tensor and its BF16 decode),
                  and the MX GEMMs on the scaled matrix cores (TFLOP/s against
                  the FP8 or FP4 peak).

The first call computes the amax; after it the three stochastic-rounding calls
run on a second stream beside the nearest-even and dequantize calls (--streams
1 runs every call in order on one stream).  After timing, the step's outputs
are checked bit for bit against the one-stream order.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--streams 2] [--no-gemm] [--no-mx] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 quantize GB/s + block-scaled GEMM TFLOP/s, % of MI355X peaks"
HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0
FP8_PEAK_TFLOPS = 5000.0
N = 8192
NBUF = 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_device(bits, torch, np):
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def time_events(fn, reps, torch):
    """Average duration (ms) of fn() over reps calls, HIP events on the
    current stream (the stream the binding launches on)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn(0)
    torch.cuda.synchronize()
    e0.record(s)
    for i in range(reps):
        fn(i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# Source files each measured kernel is built from: a traffic record taken on
# other sources is stale and reported as null.
KERNEL_SOURCES = {
    "quant": ("quantize.hip", "nvfp4_device.hpp"),
    "requant": ("quantize.hip", "nvfp4_device.hpp"),
    "dequant": ("quantize.hip", "nvfp4_device.hpp"),
    "gemm": ("gemm.hip", "nvfp4_device.hpp"),
    "mx_gemm": ("mx_gemm.hip",),
    "mx": ("mx.hip", "nvfp4_device.hpp"),
    "codec": ("mx.hip", "nvfp4_device.hpp"),
    "amax": ("quantize.hip", "nvfp4_device.hpp"),
}


def sources_of(kernel_key):
    for prefix in sorted(KERNEL_SOURCES, key=len, reverse=True):
        if kernel_key.startswith(prefix):
            return KERNEL_SOURCES[prefix]
    raise KeyError(kernel_key)


def kernel_source_hash(kernel_key):
    h = hashlib.sha256()
    for f in sources_of(kernel_key):
        with open(os.path.join(ROOT, "bit_block_scaled_quantize_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def time_rounds(cases, reps, torch, rounds):
    """Median over `rounds` rounds of time_events for each case, the cases
    interleaved within a round: the stochastic-rounding kernels run at clocks
    that the chip's power management moves by up to ~15% from one burst of
    launches to the next, so one burst per kernel is not a stable figure.
    Returns {name: (median ms, [ms of each round])}."""
    got = {k: [] for k in cases}
    for _ in range(rounds):
        for k, fn in cases.items():
            got[k].append(time_events(fn, reps, torch))
    return {k: (float(sorted(v)[len(v) // 2]), v) for k, v in got.items()}


def profile_figure(fname, kernel_key, field):
    """`field` of `kernel_key` in the committed counter summary
    profiles/`fname`, or None when absent or taken on different kernel
    sources."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    k = t.get("kernels", {}).get(kernel_key)
    if k is None or k.get("source_hash") != kernel_source_hash(kernel_key):
        return None
    return k.get(field)


def traffic_for(kernel_key):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, calibrated)."""
    return profile_figure("traffic.json", kernel_key, "hbm_bytes_per_launch")


# VALU issue peak: 256 CUs x 4 SIMDs, a wave64 instruction (64 lane-instructions)
# per SIMD every 4 cycles, at 2.4 GHz
VALU_PEAK_T_LANE_INSTR = 256 * 4 * 64 / 4 * 2.4e9 / 1e12


def valu_view(kernel_key, launch_ms):
    """The kernel against the VALU issue roofline: its counted VALU
    lane-instructions per launch (profiles/valu.json) per second of its
    launch time, against VALU_PEAK_T_LANE_INSTR; None without a matching
    counter record."""
    n = profile_figure("valu.json", kernel_key, "valu_lane_instr_per_launch")
    if n is None:
        return None
    achieved = n / (launch_ms * 1e-3) / 1e12
    return {"unit": "T VALU lane-instructions/s", "lane_instr_per_launch": n, "achieved": round(achieved, 2),
            "peak": round(VALU_PEAK_T_LANE_INSTR, 2), "frac": round(achieved / VALU_PEAK_T_LANE_INSTR, 4)}


def valu_issue_share_for(kernel_key):
    """Share of cycles the kernel's SIMDs spend issuing VALU instructions
    (SQ_INSTS_VALU x 4 / (SIMDs x cycles)): near 1, VALU issue bounds it."""
    return profile_figure("valu.json", kernel_key, "valu_issue_share")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-mx", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the step as eager launches instead of HIP graph replays")
    ap.add_argument("--streams", type=int, default=2, choices=(1, 2),
                    help="2 (default): after the first call, the three stochastic-rounding calls run "
                         "on a second stream beside the nearest-even and dequantize calls; 1: every "
                         "call in order on one stream")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--kernel-rounds", type=int, default=5,
                    help="per-kernel figures: median over this many interleaved rounds of --kernel-reps "
                         "back-to-back launches")
    ap.add_argument("--pmc-driver", action="store_true",
                    help="for rocprofv3 --pmc runs: a 1 GiB device copy (calibration), then each "
                         "step kernel alone, the column re-quantization and the MX quantize / "
                         "dequantize kernels, 3 launches each, then (unless --no-gemm) the forward "
                         "GEMM, the two 8192^3 MX GEMMs and the exact-accumulation E4M3 one twice "
                         "each, and the 8192x20480 gradient's Hadamard + column + SR quantization "
                         "(with its amax pass) twice, and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the NVFP4 path here has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_block_scaled_quantize_amd as nv
    import workloads as W

    torch.cuda.set_device(0)
    log("generating inputs")
    xs = [bf16_device(W.f32_to_bf16_bits(W.student_t((N, N), 3.0, seed=1000 + i)), torch, np)
          for i in range(NBUF)]
    dev = "cuda"
    E = N * N

    R, C = nv.NVFP4Tensor.empty(N, N, device=dev), nv.NVFP4Tensor.empty(N, N, device=dev)
    R2, C2 = nv.NVFP4Tensor.empty(N, N, device=dev), nv.NVFP4Tensor.empty(N, N, device=dev)
    # outputs of the stochastic-rounding calls of the step
    Rs, Cs = nv.NVFP4Tensor.empty(N, N, device=dev), nv.NVFP4Tensor.empty(N, N, device=dev)
    R2s, C2s = nv.NVFP4Tensor.empty(N, N, device=dev), nv.NVFP4Tensor.empty(N, N, device=dev)
    Q2d = nv.NVFP4Tensor.empty(N, N, nv.NVFP4_SCALE_2D, device=dev)
    yr = torch.empty((N, N), dtype=torch.bfloat16, device=dev)
    yc = torch.empty((N, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(nv.nvfp4_quantize_workspace_size(N, N) // 4 + 4, dtype=torch.float32, device=dev)
    amax = [torch.tensor([x.float().abs().max().item()], device=dev) for x in xs]

    ROW, COL, RC = nv.NVFP4_ROW_1D, nv.NVFP4_COL_1D, nv.NVFP4_ROW_COL_1D
    RNE, SR = nv.NVFP4_RNE, nv.NVFP4_SR
    if args.pmc_driver:
        pmc_driver(nv, torch, xs, amax, R, C, R2, C2, Q2d, yr)
        if not args.no_gemm:
            del xs
            torch.cuda.empty_cache()
            pmc_driver_gemm(nv, W, np, torch)
        print("pmc driver done", flush=True)
        return
    q1 = E * 2 + E // 2 + E // 16 + 4                    # one layout: bf16 in, codes, scales
    q2 = E * 2 + 2 * (E // 2 + E // 16) + 8              # fused row+column
    dq = E // 2 + E // 16 + 4 + E * 2                    # dequantize to bf16
    step_ops = [("quant_row_rne", ROW, RNE, q1), ("quant_row_sr", ROW, SR, q1),
                ("quant_col_rne", COL, RNE, q1), ("quant_col_sr", COL, SR, q1),
                ("quant_rowcol_rne", RC, RNE, q2), ("quant_rowcol_sr", RC, SR, q2)]
    step_bytes = sum(op[3] for op in step_ops) + 2 * dq

    amax_step = torch.zeros(1, dtype=torch.float32, device=dev)
    # The calls of a step are independent once the first has published the
    # amax.  The stochastic-rounding ones are bound by VALU issue, the others
    # by HBM, so with --streams 2 they run on a second stream (default
    # priority) beside the nearest-even and dequantize calls, which overlaps
    # the two kinds of kernel; the step ends when both streams are done.
    side = torch.cuda.Stream() if args.streams == 2 else None
    # longest first: the stream that finishes last then ends on a short call
    # (graph replays on one box: 0.334 ms with ROW, COL, fused; 0.328 with
    # fused, COL, ROW)
    sr_calls = [(RC, (R2s, C2s)), (COL, Cs), (ROW, Rs)]

    def step(i, streams=args.streams):
        x = xs[i % NBUF]
        main = torch.cuda.current_stream()
        nv.nvfp4_quantize(x, layout=ROW, round=RNE, out=R, workspace=ws, amax_out=amax_step)
        if streams == 2:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                for lay, out in sr_calls:
                    nv.nvfp4_quantize(x, layout=lay, round=SR, sr_seed=77 + i, out=out, amax_in=amax_step)
        else:
            for lay, out in sr_calls:
                nv.nvfp4_quantize(x, layout=lay, round=SR, sr_seed=77 + i, out=out, amax_in=amax_step)
        nv.nvfp4_quantize(x, layout=COL, round=RNE, out=C, amax_in=amax_step)
        nv.nvfp4_quantize(x, layout=RC, round=RNE, out=(R2, C2), amax_in=amax_step)
        nv.nvfp4_dequantize(R, out=yr)
        nv.nvfp4_dequantize(C, out=yc)
        if streams == 2:
            main.wait_stream(side)

    step_outputs = [t for q in (R, C, R2, C2, Rs, Cs, R2s, C2s) for t in (q.codes, q.scales, q.tensor_scale)]
    step_outputs += [yr, yc, amax_step]

    def timed(run):
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            run(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / args.steps

    log("eager steps")
    eager_ms = timed(step)
    if args.no_graph:
        ms = eager_ms
    else:
        # The step is a fixed sequence of launches: one HIP graph per input
        # buffer (captured from the same calls, seeds fixed per buffer)
        # replays it without the host-side gaps between launches.
        log("graph capture and timed steps")
        graphs = []
        for b in range(NBUF):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(b)
            graphs.append(g)
        torch.cuda.synchronize()
        ms = timed(lambda i: graphs[i % NBUF].replay())
    # the timed form of the step computes what the calls in order on one
    # stream compute, bit for bit
    if args.no_graph:
        step(0)
    else:
        graphs[0].replay()
    torch.cuda.synchronize()
    got = [t.clone() for t in step_outputs]
    step(0, streams=1)
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(zip(got, step_outputs)):
        if not torch.equal(a.view(torch.uint8), b.view(torch.uint8)):
            raise RuntimeError(f"step output {k} differs between the timed step and the one-stream step")
    del got
    value = step_bytes / (ms * 1e-3) / 1e9

    # ---- per-kernel durations (amax given, so each call is one kernel), as the
    # median of interleaved rounds of back-to-back launches
    log("per-kernel timing")
    reps = args.kernel_reps
    cases, nbytes = {}, {}

    def qk(lay, rnd, out):
        return lambda i: nv.nvfp4_quantize(xs[i % NBUF], layout=lay, round=rnd, sr_seed=5,
                                           amax_in=amax[i % NBUF], out=out)

    for name, lay, rnd, b in step_ops:
        out = (R2, C2) if lay == RC else (C if lay == COL else R)
        cases[name], nbytes[name] = qk(lay, rnd, out), b
    q2d = E * 2 + E // 2 + E // 256 + 4                  # 2D: one scale byte per 16 x 16 tile
    cases["quant_2d_rne"], nbytes["quant_2d_rne"] = qk(nv.NVFP4_BLK_2D, RNE, Q2d), q2d
    # dequantize and re-quantize read NVFP4 tensors: one per input buffer, and
    # one output per buffer, so consecutive launches touch different memory
    # (4 x 36 MiB in, 4 x 128 MiB or 4 x 36 MiB out) instead of re-reading one
    # tensor that stays in the 256 MB Infinity Cache
    Rb = [nv.nvfp4_quantize(xs[b], layout=ROW, round=RNE, amax_in=amax[b]) for b in range(NBUF)]
    yb = [torch.empty((N, N), dtype=torch.bfloat16, device=dev) for _ in range(NBUF)]
    cases["dequant_row_bf16"] = lambda i: nv.nvfp4_dequantize(Rb[i % NBUF], out=yb[i % NBUF])
    nbytes["dequant_row_bf16"] = dq
    # re-quantization of the row-quantized tensor along columns (not part of the step):
    # codes + scales in, codes + scales out, 1.125 B/element
    rq = 2 * (E // 2 + E // 16 + 4)
    Rq = [nv.nvfp4_quantize(xs[b], layout=ROW, round=SR, sr_seed=3 + b) for b in range(NBUF)]
    Cq = [nv.NVFP4Tensor.empty(N, N, device=dev) for _ in range(NBUF)]
    ramax = [torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(NBUF)]
    ramax_h = [torch.zeros(1, dtype=torch.float32, device=dev) for _ in range(NBUF)]
    for b in range(NBUF):
        nv.nvfp4_requantize(Rq[b], out=Cq[b], amax_out=ramax[b], workspace=ws)
        nv.nvfp4_requantize(Rq[b], out=Cq[b], hadamard=True, hadamard_seed=4, amax_out=ramax_h[b], workspace=ws)
    cases["requant_col_sr"] = lambda i: nv.nvfp4_requantize(Rq[i % NBUF], round=SR, sr_seed=6 + i,
                                                            amax_in=ramax[i % NBUF], out=Cq[i % NBUF])
    cases["requant_col_sr_hadamard"] = lambda i: nv.nvfp4_requantize(
        Rq[i % NBUF], round=SR, sr_seed=6 + i, hadamard=True, hadamard_seed=4, amax_in=ramax_h[i % NBUF],
        out=Cq[i % NBUF])
    nbytes["requant_col_sr"] = nbytes["requant_col_sr_hadamard"] = rq
    # the amax pass: the row quantize with its amax computed, less the kernel alone
    cases["quant_row_rne_with_amax"] = lambda i: nv.nvfp4_quantize(xs[i % NBUF], layout=ROW, out=R, workspace=ws)
    timed_k = time_rounds(cases, reps, torch, args.kernel_rounds)
    del Rb, yb, Rq, Cq
    kern = {k: dict(ms=timed_k[k][0], ms_rounds=[round(x, 5) for x in timed_k[k][1]], bytes=nbytes[k])
            for k in nbytes}
    amax_ms = timed_k["quant_row_rne_with_amax"][0] - timed_k["quant_row_rne"][0]
    kern["amax_pass"] = dict(ms=amax_ms, bytes=E * 2)
    for k, v in kern.items():
        v["gbs"] = v["bytes"] / (v["ms"] * 1e-3) / 1e9
        v["frac_hbm"] = v["gbs"] / HBM_PEAK_GBS
    # time share in the step: one amax pass plus one kernel per call
    share = {k: kern[k]["ms"] for k, *_ in step_ops}
    share["amax_pass"] = amax_ms
    share["dequant_row_bf16"] = 2 * kern["dequant_row_bf16"]["ms"]
    dom = max((k for k in share if k != "amax_pass"), key=lambda k: share[k])
    dk = kern[dom]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dk["gbs"], 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(dk["frac_hbm"], 4), "traffic": traffic_for(dom),
                "avg_launch_ms": round(dk["ms"], 5), "algorithmic_bytes_per_launch": dk["bytes"],
                "timing": f"median over {args.kernel_rounds} interleaved rounds of the average of "
                          f"{args.kernel_reps} back-to-back launches (HIP events on the launch stream)",
                "avg_launch_ms_rounds": dk["ms_rounds"],
                "valu_issue_share": valu_issue_share_for(dom),
                "valu_view": valu_view(dom, dk["ms"])}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "quantize_8192x8192_bf16_student_t3", "rows": N, "cols": N,
                   "input": "bf16", "step": [k for k, *_ in step_ops] + ["dequant_row_bf16",
                                                                       "dequant_col_bf16"],
                   "amax": "computed once per tensor by the first call (amax_out) and reused by the others (amax_in)",
                   "bytes_per_step": step_bytes, "input_buffers": NBUF,
                   "launch": "eager" if args.no_graph else "hip_graph_replay",
                   "streams": args.streams,
                   "eager_ms_per_step": round(eager_ms, 4)},
        "roofline": roofline,
        "kernels": {k: {"ms": round(v["ms"], 5), "GB/s": round(v["gbs"], 1),
                        "frac_hbm": round(v["frac_hbm"], 4), "hbm_bytes": traffic_for(k),
                        **({"ms_rounds": v["ms_rounds"]} if "ms_rounds" in v else {})} for k, v in kern.items()},
    }

    if not args.no_mx:
        result["mx"] = bench_mx_quant(nv, torch, xs, reps, args.kernel_rounds)
    del xs
    torch.cuda.empty_cache()
    if not args.no_mx:
        result["mx"].update(bench_mx_codec(nv, W, np, torch, reps))
        if not args.no_gemm:
            result["mx"].update(bench_mx_gemm(nv, W, np, torch, reps=max(3, reps // 4)))
    if not args.no_gemm:
        extra = {}
        result["gemm"] = bench_gemm(nv, W, np, torch, reps=max(3, reps // 4), kern_extra=extra)
        for k, v in extra.items():
            gbs = v["bytes"] / (v["ms"] * 1e-3) / 1e9
            result["kernels"][k] = {"ms": round(v["ms"], 5), "GB/s": round(gbs, 1),
                                    "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "hbm_bytes": traffic_for(k),
                                    "ms_rounds": v["ms_rounds"]}

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(np, W)
        if not args.no_gemm:
            result["gemm"]["cpu_oracle_forward_8192x20480x5120_sampled"] = cpu_oracle_gemm(np, W)
    print(json.dumps(result), flush=True)


def pmc_driver(nv, torch, xs, amax, R, C, R2, C2, Q2d, yr):
    """Kernel sequence for hardware-counter runs: the calibration copy first
    (1 GiB read + 1 GiB written by torch's copy kernel, its source evicted
    from the caches by a 1 GiB fill of another buffer before each copy), then
    every step kernel alone (amax given), three launches each, on distinct
    inputs."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    flush = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        flush.fill_(2)
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst, flush
    ROW, COL, RC, B2 = nv.NVFP4_ROW_1D, nv.NVFP4_COL_1D, nv.NVFP4_ROW_COL_1D, nv.NVFP4_BLK_2D
    for lay, rnd, out in [(ROW, 0, R), (ROW, 1, R), (COL, 0, C), (COL, 1, C), (RC, 0, (R2, C2)),
                          (RC, 1, (R2, C2)), (B2, 0, Q2d)]:
        for i in range(3):
            nv.nvfp4_quantize(xs[i], layout=lay, round=rnd, sr_seed=5, amax_in=amax[i], out=out)
        torch.cuda.synchronize()
    for i in range(3):
        nv.nvfp4_dequantize(R, out=yr)
    torch.cuda.synchronize()
    # re-quantization along columns of the row-quantized tensor (SR, amax given)
    Rq = nv.nvfp4_quantize(xs[0], round=1, sr_seed=3)
    ramax = torch.zeros(1, dtype=torch.float32, device="cuda")
    nv.nvfp4_requantize(Rq, out=C, amax_out=ramax)
    torch.cuda.synchronize()
    for i in range(3):
        nv.nvfp4_requantize(Rq, round=1, sr_seed=6 + i, amax_in=ramax, out=C)
    torch.cuda.synchronize()
    # MX quantize / dequantize
    E4, E2 = nv.NVFP4_MX_E4M3, nv.NVFP4_MX_E2M1
    q4, q2 = nv.MXTensor.empty(N, N, E4), nv.MXTensor.empty(N, N, E2)
    for lay, elem, rnd, q in [(ROW, E4, 0, q4), (ROW, E4, 1, q4), (COL, E4, 1, q4), (ROW, E2, 0, q2), (ROW, E2, 1, q2)]:
        for i in range(3):
            nv.nvfp4_mx_quantize(xs[i], layout=lay, elem=elem, round=rnd, sr_seed=5, out=q)
        torch.cuda.synchronize()
    for i in range(3):
        nv.nvfp4_mx_dequantize(q4, out=yr)
    torch.cuda.synchronize()


def pmc_driver_gemm(nv, W, np, torch):
    """Counter runs of the block-scaled GEMM: the forward shape (8192 x 20480
    x 5120, BF16 out, 2D-scaled weights), two launches."""
    X = nv.nvfp4_quantize(bf16_device(W.f32_to_bf16_bits(W.student_t((8192, 5120), 3.0, seed=4000)), torch, np))
    Wt = nv.nvfp4_quantize(bf16_device(W.f32_to_bf16_bits(W.normal((20480, 5120), 0.02, seed=4001)), torch, np),
                           layout=nv.NVFP4_BLK_2D)
    Y = torch.empty((8192, 20480), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(2):
        nv.nvfp4_gemm(X, Wt, out=Y)
    torch.cuda.synchronize()
    del X, Wt, Y
    # MX GEMMs 8192^3, FP32 out (native; then E4M3 with exact accumulation)
    for elem in (nv.NVFP4_MX_E4M3, nv.NVFP4_MX_E2M1):
        A = nv.nvfp4_mx_quantize(bf16_device(W.f32_to_bf16_bits(W.student_t((8192, 8192), 3.0, seed=7100)), torch, np),
                                 elem=elem)
        B = nv.nvfp4_mx_quantize(bf16_device(W.f32_to_bf16_bits(W.student_t((8192, 8192), 3.0, seed=7200)), torch, np),
                                 elem=elem)
        C = torch.empty((8192, 8192), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        for _ in range(2):
            nv.nvfp4_mx_gemm(A, B, out=C)
        torch.cuda.synchronize()
        if elem == nv.NVFP4_MX_E4M3:
            for _ in range(2):
                nv.nvfp4_mx_gemm(A, B, out=C, accum=nv.NVFP4_MX_ACC_EXACT)
            torch.cuda.synchronize()
        del A, B, C
    # the 8192 x 20480 gradient's transformed amax (down columns) and its
    # Hadamard + column + SR quantization, two calls
    dy = bf16_device(W.f32_to_bf16_bits(W.with_spikes(W.normal((8192, 20480), 1.0, seed=5000), 1e-4, 100.0,
                                                      seed=5001)), torch, np)
    for i in range(2):
        nv.nvfp4_quantize(dy, layout=nv.NVFP4_COL_1D, round=nv.NVFP4_SR, sr_seed=5100 + i, hadamard=True,
                          hadamard_seed=5200)
    torch.cuda.synchronize()
    del dy


def bench_gemm(nv, W, np, torch, reps, kern_extra=None):
    """Block-scaled GEMM throughput at the forward, weight-gradient and MoE
    shapes; operands are quantized on the GPU from seeded inputs."""
    out = {}

    def gen(shape, seed, kind):
        if kind == "t3":
            x = W.student_t(shape, 3.0, seed=seed)
        elif kind == "w":
            x = W.normal(shape, 0.02, seed=seed)
        else:
            x = W.with_spikes(W.normal(shape, 1.0, seed=seed), 1e-4, 100.0, seed=seed + 1)
        return bf16_device(W.f32_to_bf16_bits(x), torch, np)

    def entry(name, flop, ms):
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                     "frac_fp16_mfma_peak": round(tf / FP16_PEAK_TFLOPS, 4),
                     "frac_fp4_mfma_peak": round(tf / FP4_PEAK_TFLOPS, 4)}

    log("gemm: 256^3")
    # M = N = K = 256, FP32 N(0,1) with 0.1% x50 outliers; A along rows, B
    # (K x N) along K, RNE, FP32 out: quantize both operands and multiply
    # (latency-bound; one launch per call, amax computed by each quantize)
    a = torch.from_numpy(W.with_spikes(W.normal((256, 256), 1.0, seed=1), 1e-3, 50.0, seed=2)).cuda()
    b = torch.from_numpy(W.with_spikes(W.normal((256, 256), 1.0, seed=3), 1e-3, 50.0, seed=4)).cuda()
    Aq = nv.nvfp4_quantize(a)
    Bq = nv.nvfp4_quantize(b, layout=nv.NVFP4_COL_1D)
    C = torch.empty((256, 256), dtype=torch.float32, device="cuda")
    entry("gemm_256x256x256_f32", 2 * 256 ** 3, time_events(lambda i: nv.nvfp4_gemm(Aq, Bq, out=C), reps, torch))

    ws = torch.empty((nv.nvfp4_quantize_workspace_size(256, 256) + 15) // 16 * 4, dtype=torch.float32,
                     device="cuda")

    def c1(i):
        nv.nvfp4_quantize(a, out=Aq, workspace=ws)
        nv.nvfp4_quantize(b, layout=nv.NVFP4_COL_1D, out=Bq, workspace=ws)
        nv.nvfp4_gemm(Aq, Bq, out=C)
    out["gemm_256x256x256_f32"]["quantize_both_and_gemm_ms"] = round(time_events(c1, reps, torch), 4)
    del a, b, Aq, Bq, C, ws

    log("gemm: forward")
    X = nv.nvfp4_quantize(gen((8192, 5120), 4000, "t3"))
    Wt = nv.nvfp4_quantize(gen((20480, 5120), 4001, "w"), layout=nv.NVFP4_BLK_2D)
    Y = torch.empty((8192, 20480), dtype=torch.bfloat16, device="cuda")
    entry("forward_8192x20480x5120_bf16", 2 * 8192 * 20480 * 5120,
          time_events(lambda i: nv.nvfp4_gemm(X, Wt, out=Y), reps, torch))
    del X, Wt, Y
    log("gemm: wgrad")
    kw = dict(layout=nv.NVFP4_COL_1D, round=nv.NVFP4_SR, hadamard=True, hadamard_seed=5200)
    dy = gen((8192, 20480), 5000, "spiky")
    dYq = nv.nvfp4_quantize(dy, sr_seed=5100, **kw)
    if kern_extra is not None:
        # the gradient's own quantization (320 MiB, larger than the Infinity
        # Cache): 16-point Hadamard along tokens, column blocks, SR; with the
        # amax given, and with the transformed tensor's amax computed first
        eg = 8192 * 20480
        amax_h = torch.zeros(1, dtype=torch.float32, device="cuda")
        ws_h = torch.empty((nv.nvfp4_quantize_workspace_size(8192, 20480) + 15) // 16 * 4,
                           dtype=torch.float32, device="cuda")
        nv.nvfp4_quantize(dy, sr_seed=5100, amax_out=amax_h, out=dYq, workspace=ws_h, **kw)
        qb = eg * 2 + eg // 2 + eg // 16 + 4
        tg = time_rounds({
            "quant_col_sr_hadamard_8192x20480":
                lambda i: nv.nvfp4_quantize(dy, sr_seed=5100 + i, amax_in=amax_h, out=dYq, **kw),
            "quant_col_sr_hadamard_8192x20480_with_amax":
                lambda i: nv.nvfp4_quantize(dy, sr_seed=5100 + i, out=dYq, workspace=ws_h, **kw)},
            10, torch, 3)
        for k, (ms_k, rounds_k) in tg.items():
            kern_extra[k] = dict(ms=ms_k, bytes=qb, ms_rounds=[round(x, 5) for x in rounds_k])
        nv.nvfp4_quantize(dy, sr_seed=5100, out=dYq, workspace=ws_h, **kw)
        del ws_h, amax_h
    del dy
    Xq = nv.nvfp4_quantize(gen((8192, 5120), 5002, "spiky"), sr_seed=5101, **kw)
    dW = torch.empty((20480, 5120), dtype=torch.float32, device="cuda")
    entry("wgrad_20480x5120x8192_f32", 2 * 20480 * 5120 * 8192,
          time_events(lambda i: nv.nvfp4_gemm(dYq, Xq, out=dW), reps, torch))
    del dYq, Xq, dW
    torch.cuda.empty_cache()

    log("gemm: moe")
    E, Hd, F, T = 32, 7168, 2048, 16384
    counts = W.zipf_expert_counts(E, T, 4, 1.1)
    offs, token = W.moe_routing(counts, T)
    Xq = nv.nvfp4_quantize(gen((T, Hd), 6000, "t3"))
    idx = torch.from_numpy(token).cuda()
    A = nv.NVFP4Tensor(Xq.codes.index_select(0, idx), Xq.scales.index_select(0, idx),
                       Xq.tensor_scale, int(offs[-1]), Hd)

    def stacked(rows, cols, seed):
        Wq = nv.NVFP4Tensor.empty(E * rows, cols, nv.NVFP4_SCALE_2D, n_scales=E)
        for e in range(E):
            q = nv.nvfp4_quantize(gen((rows, cols), seed + e, "w"), layout=nv.NVFP4_BLK_2D)
            Wq.codes[e * rows:(e + 1) * rows].copy_(q.codes)
            Wq.scales[e * rows // 16:(e + 1) * rows // 16].copy_(q.scales)
            Wq.tensor_scale[e:e + 1].copy_(q.tensor_scale)
        return Wq

    W1 = stacked(2 * F, Hd, 6100)
    W2 = stacked(Hd, F, 6200)
    offs_d = torch.from_numpy(offs).cuda()
    H = torch.empty((int(offs[-1]), F), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((int(offs[-1]), Hd), dtype=torch.bfloat16, device="cuda")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    Hq = nv.NVFP4Tensor.empty(int(offs[-1]), F)
    rows = int(offs[-1])
    up_flop = 2 * rows * 2 * F * Hd
    down_flop = 2 * rows * Hd * F
    up_ms = time_events(lambda i: nv.nvfp4_grouped_gemm(A, offs_d, W1, E, epilogue=nv.NVFP4_EPI_SWIGLU,
                                                        out=H, amax_out=amax), reps, torch)
    q_ms = time_events(lambda i: nv.nvfp4_quantize(H, amax_in=amax, out=Hq), reps, torch)
    down_ms = time_events(lambda i: nv.nvfp4_grouped_gemm(Hq, offs_d, W2, E, out=Y), reps, torch)
    entry("moe_up_swiglu_65536x4096x7168", up_flop, up_ms)
    entry("moe_down_65536x7168x2048", down_flop, down_ms)
    entry("moe_expert_forward_total", up_flop + down_flop, up_ms + q_ms + down_ms)
    out["moe_expert_forward_total"]["quantize_h_ms"] = round(q_ms, 4)
    return out


def _gbs(name, nbytes, ms):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {name: {"ms": round(ms, 5), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                   "bytes": nbytes, "hbm_bytes": traffic_for(name)}}


def bench_mx_quant(nv, torch, xs, reps, rounds):
    """MX quantize / dequantize of the step's 8192 x 8192 BF16 tensors (no
    amax pass: MX scales are per block only).  Bytes: input + codes + E8M0
    scales (quantize); codes + scales + BF16 output (dequantize)."""
    log("mx: quantize")
    E = N * N
    E4, E2 = nv.NVFP4_MX_E4M3, nv.NVFP4_MX_E2M1
    out = {}
    q = {E4: nv.MXTensor.empty(N, N, E4), E2: nv.MXTensor.empty(N, N, E2)}
    code_bytes = {E4: E, E2: E // 2}
    cases, nbytes = {}, {}
    for name, lay, elem, rnd in [("mx_e4m3_row_rne", nv.NVFP4_ROW_1D, E4, nv.NVFP4_RNE),
                                 ("mx_e4m3_row_sr", nv.NVFP4_ROW_1D, E4, nv.NVFP4_SR),
                                 ("mx_e4m3_col_rne", nv.NVFP4_COL_1D, E4, nv.NVFP4_RNE),
                                 ("mx_e4m3_col_sr", nv.NVFP4_COL_1D, E4, nv.NVFP4_SR),
                                 ("mx_e2m1_row_rne", nv.NVFP4_ROW_1D, E2, nv.NVFP4_RNE),
                                 ("mx_e2m1_row_sr", nv.NVFP4_ROW_1D, E2, nv.NVFP4_SR),
                                 ("mx_e2m1_col_sr", nv.NVFP4_COL_1D, E2, nv.NVFP4_SR)]:
        cases[name] = (lambda lay, elem, rnd: lambda i: nv.nvfp4_mx_quantize(
            xs[i % NBUF], layout=lay, elem=elem, round=rnd, sr_seed=9 + i, out=q[elem]))(lay, elem, rnd)
        nbytes[name] = E * 2 + code_bytes[elem] + E // 32
    # dequantize: one MX tensor and one output per input buffer (rotated)
    ys = [torch.empty((N, N), dtype=torch.bfloat16, device="cuda") for _ in range(NBUF)]
    qs = {}
    for name, elem in [("mx_dequant_e4m3_bf16", E4), ("mx_dequant_e2m1_bf16", E2)]:
        qs[elem] = [nv.nvfp4_mx_quantize(xs[b], elem=elem) for b in range(NBUF)]
        cases[name] = (lambda elem: lambda i: nv.nvfp4_mx_dequantize(qs[elem][i % NBUF], out=ys[i % NBUF]))(elem)
        nbytes[name] = code_bytes[elem] + E // 32 + E * 2
    timed = time_rounds(cases, reps, torch, rounds)
    for name in cases:
        out.update(_gbs(name, nbytes[name], timed[name][0]))
        out[name]["ms_rounds"] = [round(x, 5) for x in timed[name][1]]
    del qs, ys
    return out


def bench_mx_codec(nv, W, np, torch, reps):
    """The 8.25-bit expert-output codec at the MoE output shape (65536 x 7168
    BF16, the down-projection's output of 16384 tokens x top-4): MXFP8 row
    encode (8 + 8/32 bits per number) and the BF16 decode.  Student-t(3)
    rows (an 8192-row seeded block repeated 8 times)."""
    log("mx: codec")
    rows, cols = 65536, 7168
    blk = bf16_device(W.f32_to_bf16_bits(W.student_t((8192, cols), 3.0, seed=7000)), torch, np)
    Y = blk.repeat(rows // 8192, 1)
    del blk
    E = rows * cols
    q = nv.MXTensor.empty(rows, cols, nv.NVFP4_MX_E4M3)
    y = torch.empty_like(Y)
    out = {}
    ms = time_events(lambda i: nv.nvfp4_mx_quantize(Y, out=q), reps, torch)
    out.update(_gbs("codec_encode_65536x7168", E * 2 + E + E // 32, ms))
    ms = time_events(lambda i: nv.nvfp4_mx_dequantize(q, out=y), reps, torch)
    out.update(_gbs("codec_decode_65536x7168", E + E // 32 + E * 2, ms))
    out["codec_encode_65536x7168"]["bits_per_number"] = 8.25
    out["codec_encode_65536x7168"]["payload_bytes"] = E + E // 32
    del Y, y, q
    torch.cuda.empty_cache()
    return out


def bench_mx_gemm(nv, W, np, torch, reps):
    """MX GEMMs, operands MX-quantized on the GPU from seeded BF16 data (SR):
    the native path on the scaled matrix cores (against the FP8 or FP4 peak)
    and the exact path (exact products, binary32 sums, on the BF16 matrix
    cores: against the BF16 peak).  For the native path the line also carries
    its error relative to sum |a b| over the whole output: |native - exact| /
    sum |a b|, where the exact path is within 1e-5 sum |a b| of the exact
    product (its parity tests) and sum |a b| is the exact path's GEMM of the
    operands with every sign bit cleared."""
    out = {}

    def mxq(shape, seed, elem):
        x = bf16_device(W.f32_to_bf16_bits(W.student_t(shape, 3.0, seed=seed)), torch, np)
        return nv.nvfp4_mx_quantize(x, elem=elem, round=nv.NVFP4_SR, sr_seed=seed + 1)

    def magnitude(q, elem):
        # the same MX tensor with every element's sign bit cleared
        mask = 0x7F if elem == nv.NVFP4_MX_E4M3 else 0x77
        return nv.MXTensor(torch.bitwise_and(q.codes, mask), q.scales, q.rows, q.cols, q.elem)

    EX = nv.NVFP4_MX_ACC_EXACT
    for elem, tag, peak in [(nv.NVFP4_MX_E4M3, "e4m3", FP8_PEAK_TFLOPS), (nv.NVFP4_MX_E2M1, "e2m1", FP4_PEAK_TFLOPS)]:
        for (M, Nn, K, dt) in [(8192, 8192, 8192, torch.float32), (20480, 5120, 8192, torch.float32)]:
            log(f"mx gemm {tag} {M}x{Nn}x{K}")
            A, B = mxq((M, K), 7100, elem), mxq((Nn, K), 7200, elem)
            C = torch.empty((M, Nn), dtype=dt, device="cuda")
            Ce = torch.empty((M, Nn), dtype=dt, device="cuda")
            ms = time_events(lambda i: nv.nvfp4_mx_gemm(A, B, out=C), reps, torch)
            ms_x = time_events(lambda i: nv.nvfp4_mx_gemm(A, B, out=Ce, accum=EX), reps, torch)
            tf = 2 * M * Nn * K / (ms * 1e-3) / 1e12
            tf_x = 2 * M * Nn * K / (ms_x * 1e-3) / 1e12
            nv.nvfp4_mx_gemm(magnitude(A, elem), magnitude(B, elem), out=C, accum=EX)   # C = sum |a b|
            Cn = nv.nvfp4_mx_gemm(A, B)
            rel = ((Cn.double() - Ce.double()).abs() / C.double().clamp_min(1e-300)).flatten()
            out[f"mx_gemm_{tag}_{M}x{Nn}x{K}"] = {
                "ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_peak": round(tf / peak, 4),
                "peak_TFLOP/s": peak,
                "native_error_vs_sum_abs_ab": {"max": float(rel.max()), "median": float(rel.median()),
                                               "meets_1e-5": bool(rel.max() <= 1e-5)},
                "exact": {"ms": round(ms_x, 4), "TFLOP/s": round(tf_x, 1),
                          "frac_bf16_peak": round(tf_x / FP16_PEAK_TFLOPS, 4)}}
            del A, B, C, Ce, Cn, rel
            torch.cuda.empty_cache()
    return out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(np, W, rows=N):
    """The oracle on rows 0 .. rows-1 of the 8192 x 8192 step input (by default
    the whole tensor): the same quantize calls and dequantizations as the
    step, first as single oracle calls on one core (about 13 s on the GPU
    box's host), then band by band on every core this process may use
    (oracle/banded.py: the unchanged oracle called once per independent band
    in threads), whose outputs must equal the single-core ones byte for
    byte.  `value` is the all-core rate; the single-core rate is reported
    beside it."""
    import oracle as O
    from oracle import banded as OB
    x = W.f32_to_bf16_bits(W.student_t((N, N), 3.0, seed=1000))[:rows].copy()
    E = rows * N

    def run(quantize, dequantize, **kw):
        outs = []
        for lay in (O.ROW_1D, O.COL_1D):
            for rnd in (O.RNE, O.SR):
                outs.append(quantize(x, O.BF16, lay, rnd, sr_seed=77, **kw))
        for rnd in (O.RNE, O.SR):
            qr, qc = quantize(x, O.BF16, O.ROW_COL_1D, rnd, sr_seed=77, **kw)
            outs += [qr, qc]
        outs.append(dequantize(outs[0], O.BF16, **kw))
        outs.append(dequantize(outs[2], O.BF16, **kw))
        return outs

    t0 = time.perf_counter()
    single = run(O.quantize, O.dequantize)
    t_single = time.perf_counter() - t0
    threads = OB.default_threads()
    t0 = time.perf_counter()
    multi = run(OB.quantize, OB.dequantize, threads=threads)
    t_multi = time.perf_counter() - t0
    for a, b in zip(single, multi):
        if isinstance(a, np.ndarray):
            same = np.array_equal(a, b)
        else:
            same = a.ts == b.ts and np.array_equal(a.codes, b.codes) and np.array_equal(a.scales, b.scales)
        if not same:
            raise RuntimeError("the banded oracle differs from the single-call oracle")
    q1 = E * 2 + E // 2 + E // 16 + 4
    q2 = E * 2 + 2 * (E // 2 + E // 16) + 8
    dq = E // 2 + E // 16 + 4 + E * 2
    b = 4 * q1 + 2 * q2 + 2 * dq
    return {"value": round(b / t_multi / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single_core_value": round(b / t_single / 1e9, 4),
            "cpu_model": cpu_model(), "host_cpus_visible": os.cpu_count(),
            "sample": f"rows 0..{rows - 1} of the {N}x{N} step input"
                      f"{' (the whole tensor)' if rows == N else ''}: the step's quantize and "
                      f"dequantize calls; {t_single:.1f} s as single oracle calls on one core, "
                      f"{t_multi:.2f} s band by band on {threads} threads (identical outputs)"}


def cpu_oracle_gemm(np, W, n_entries=8192):
    """The oracle GEMM (exact dequantization, float64 dot products) on sampled
    output entries of the forward shape 8192 x 20480 x 5120 (X Student-t(3)
    row blocks, W N(0, 0.02) 16x16 blocks).  The operand rows
    the entries need are quantized by the oracle beforehand (not timed); the
    per-entry time is extrapolated to the whole output.  Timed on one core,
    then with the entries split over every core this process may use."""
    import oracle as O
    from oracle import banded as OB
    M, Nn, K = 8192, 20480, 5120
    x = W.f32_to_bf16_bits(W.student_t((M, K), 3.0, seed=4000))
    w = W.f32_to_bf16_bits(W.normal((Nn, K), 0.02, seed=4001))
    g = W.rng(4002)
    # columns from 128 random 16-row bands of W, so the untimed operand
    # quantization stays small
    mi = g.integers(0, M, n_entries)
    ni = 16 * g.choice(Nn // 16, 128, replace=False)[g.integers(0, 128, n_entries)] + g.integers(0, 16, n_entries)
    mu, ml = np.unique(mi, return_inverse=True)
    A = O.quantize(np.ascontiguousarray(x[mu]), O.BF16, O.ROW_1D, amax_in=O.amax(x, O.BF16, O.ROW_1D))
    bands = np.unique(ni // 16)
    B = O.quantize(np.concatenate([w[16 * b:16 * b + 16] for b in bands]), O.BF16, O.BLK_2D,
                   amax_in=O.amax(w, O.BF16, O.BLK_2D))
    nl = np.searchsorted(bands, ni // 16) * 16 + ni % 16
    t0 = time.perf_counter()
    c1, _ = O.gemm(A, B, entries=(ml, nl))
    dt = time.perf_counter() - t0
    threads = OB.default_threads()
    t0 = time.perf_counter()
    cn, _ = OB.gemm_entries(A, B, ml, nl, threads=threads)
    dtn = time.perf_counter() - t0
    if not np.array_equal(c1, cn):
        raise RuntimeError("the threaded oracle GEMM differs from the single-call one")
    full_s = dt / n_entries * M * Nn
    full_n = dtn / n_entries * M * Nn
    return {"entries": n_entries, "seconds": round(dtn, 3), "cores": threads, "kind": "oracle",
            "extrapolated_full_seconds": round(full_n, 1),
            "extrapolated_TFLOP/s": round(2 * M * Nn * K / full_n / 1e12, 6),
            "single_core_seconds": round(dt, 3),
            "single_core_extrapolated_full_seconds": round(full_s, 1)}


if __name__ == "__main__":
    main()
