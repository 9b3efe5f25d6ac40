"""Shared helpers of the GPU parity tests: move seeded host inputs to the
device, run the HIP path through the Python binding of the C ABI, and bring
results back as numpy arrays for comparison with the oracle."""
import numpy as np
import pytest
import torch

import oracle as O


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import bit_block_scaled_quantize_amd as nv  # raises if libnvfp4.so is missing
    return nv


def to_device(x, pad_to=None):
    """numpy float32 or uint16 (bf16 bits) [r, c] -> device tensor.  With
    pad_to, the row stride is pad_to elements (a strided view)."""
    r, c = x.shape
    cols = c if pad_to is None else pad_to
    if x.dtype == np.uint16:
        buf = np.zeros((r, cols), dtype=np.uint16)
        buf[:, :c] = x
        t = torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        buf = np.zeros((r, cols), dtype=np.float32)
        buf[:, :c] = x
        t = torch.from_numpy(buf).cuda()
    return t[:, :c]


def q_to_host(q):
    """NVFP4Tensor (device) -> oracle.QTensor (host)."""
    torch.cuda.synchronize()
    return O.QTensor(q.codes.cpu().numpy(), q.scales.cpu().numpy(), float(q.tensor_scale[0].item()),
                     q.rows, q.cols, q.scale_mode)


def q_to_device(q, nv):
    """oracle.QTensor (host) -> NVFP4Tensor (device)."""
    return nv.NVFP4Tensor(torch.from_numpy(np.ascontiguousarray(q.codes)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(q.scales)).cuda(),
                          torch.tensor([q.ts], dtype=torch.float32, device="cuda"),
                          q.rows, q.cols, q.scale_mode)


def assert_q_equal(got, ref, what=""):
    assert got.ts == ref.ts, f"{what}: tensor scale {got.ts!r} != {ref.ts!r}"
    if not np.array_equal(got.scales, ref.scales):
        bad = np.argwhere(got.scales != ref.scales)
        raise AssertionError(f"{what}: {len(bad)} scale bytes differ, first at {bad[0].tolist()} "
                             f"gpu={got.scales[tuple(bad[0])]:#x} oracle={ref.scales[tuple(bad[0])]:#x}")
    if not np.array_equal(got.codes, ref.codes):
        bad = np.argwhere(got.codes != ref.codes)
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at {bad[0].tolist()} "
                             f"gpu={got.codes[tuple(bad[0])]:#04x} oracle={ref.codes[tuple(bad[0])]:#04x}")


def bf16_tensor_to_bits(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gemm_tol(Cref, Wref, bf16_out):
    """|gpu - oracle| <= 1e-5 * sum|a b| per element; bf16 outputs add half a
    bf16 ulp of the reference value (the final rounding to bf16)."""
    tol = 1e-5 * Wref
    if bf16_out:
        a = np.abs(Cref)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        tol = tol + np.where(a > 0, 2.0 ** (e - 8), 0.0)
    return tol
