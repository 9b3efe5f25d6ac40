"""MI355X (gfx950) NVFP4: block-scaled 4-bit quantization and block-scaled
GEMMs as hand-written HIP kernels behind a C ABI (include/nvfp4.h).

The Python names mirror the C entry points; see nvfp4.py."""
from .nvfp4 import (  # noqa: F401
    NVFP4Error, NVFP4Tensor, lib,
    NVFP4_F32, NVFP4_BF16, NVFP4_ROW_1D, NVFP4_COL_1D, NVFP4_ROW_COL_1D, NVFP4_BLK_2D,
    NVFP4_RNE, NVFP4_SR, NVFP4_EPI_NONE, NVFP4_EPI_SWIGLU, NVFP4_SCALE_1D, NVFP4_SCALE_2D,
    nvfp4_quantize, nvfp4_quantize_noalloc, nvfp4_quantize_workspace_size, nvfp4_requantize, nvfp4_dequantize, nvfp4_gemm, nvfp4_gemm_workspace_size,
    nvfp4_grouped_gemm,
    MXTensor, NVFP4_MX_E4M3, NVFP4_MX_E2M1, NVFP4_MX_ACC_NATIVE, NVFP4_MX_ACC_EXACT,
    nvfp4_mx_quantize, nvfp4_mx_dequantize,
    nvfp4_mx_gemm, nvfp4_mx_gemm_workspace_size,
)
