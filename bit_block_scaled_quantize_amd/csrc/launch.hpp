// Internal host interface between the C-ABI layer (nvfp4_api.hip) and the
// kernel translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace nvfp4 {

enum { kLayoutRow = 0, kLayoutCol = 1, kLayoutRowCol = 2, kLayout2D = 3 };

// MX element formats (nvfp4_mx_elem).
enum { kMxE4M3 = 0, kMxE2M1 = 1 };

// Upper bound on the per-workgroup partial maxima of one amax pass; the
// quantize workspace holds exactly these floats, and every quantize
// workgroup reduces them in its prologue.
constexpr int64_t kMaxPartials = 512;
constexpr size_t kQuantWorkspaceBytes = (size_t)kMaxPartials * sizeof(float);

struct QOut {
    uint8_t* codes;
    uint8_t* scales;
    float* ts;
};

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           int layout, bool sr, uint64_t seed, bool rht, uint64_t hseed,
                           const float* amax_in, float* amax_out, const QOut* out, float* ws,
                           hipStream_t s);

// COL_1D re-quantization of a row-blocked NVFP4 tensor (rows x cols, both
// multiples of 16); out is cols x rows.
hipError_t launch_requantize(const uint8_t* icodes, const uint8_t* iscales, const float* its,
                             int64_t rows, int64_t cols, bool sr, uint64_t seed, bool rht,
                             uint64_t hseed, const float* amax_in, float* amax_out, const QOut* out,
                             float* ws, hipStream_t s);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts,
                             int64_t rows, int64_t cols, bool scale_2d, void* y, bool bf16,
                             int64_t ld, hipStream_t s);

// One GEMM operand as the kernels see it.
struct Operand {
    const uint8_t* codes;   // rows x K/2
    const uint8_t* scales;  // 1D: rows x K/16; 2D: rows/16 x K/16
    const float* ts;        // tensor scale(s)
    int scale_2d;
};

// C (M x N, ldc) = A * B^T; c_bf16 selects the output type.  swiglu: N = 2F,
// C (M x F, BF16) = gate * sigmoid(gate) * up with gate = columns [0, F) and
// up = columns [F, 2F) of A * B^T.
hipError_t launch_gemm(const Operand& A, const Operand& B, int64_t M, int64_t N, int64_t K,
                       void* C, bool c_bf16, int64_t ldc, bool swiglu, void* ws, size_t ws_bytes,
                       hipStream_t s);

// Split of a plain GEMM's last round of tiles along K (workspace for the
// parts' accumulators: `bytes`; split 1: none).  The tiles after t_main, a
// round that would leave compute units idle, are each computed in `split`
// parts by otherwise idle units and summed in part order by a second kernel.
struct GemmSplit {
    int64_t t_main;
    int split;
    int64_t bytes;
};
constexpr int64_t kMaxTailSplit = 8;
GemmSplit gemm_split_plan(int64_t M, int64_t N, int64_t K, bool swiglu, int cus);
// Compute units of the current device.
hipError_t device_cus(int& cus);

// Grouped GEMM over G groups (see nvfp4_grouped_gemm).  n_per_group = rows of
// one group's weight matrix; swiglu halves the output width.
hipError_t launch_grouped_gemm(int G, const Operand& A, const int64_t* offsets, int64_t total_rows,
                               const Operand& B, int64_t n_per_group, int64_t K, void* C,
                               bool c_bf16, int64_t ldc, bool swiglu, float* amax_out,
                               hipStream_t s);

// MX quantization (layout kLayoutRow or kLayoutCol; the block dimension is a
// multiple of 32) into codes / E8M0 scales of the output orientation.
hipError_t launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld, int layout,
                              int elem, bool sr, uint64_t seed, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int elem, int64_t rows,
                                int64_t cols, void* y, bool bf16, int64_t ld, hipStream_t s);

// C (M x N, ldc) = A * B^T for MX operands of one element format; K % 64 == 0.
// exact: every product exact and binary32 accumulation (BF16 matrix cores on
// exactly rescaled elements) instead of the scaled matrix cores.
hipError_t launch_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int elem, int64_t M, int64_t N, int64_t K, void* C,
                          bool c_bf16, int64_t ldc, bool exact, void* ws, size_t ws_bytes, hipStream_t s);
// The MX GEMM's split plan (full-line kernels: K % 1024 == 0).
GemmSplit mx_gemm_split_plan(int64_t M, int64_t N, int64_t K, double tile_us, int cus);
// A lone last-round tile's time per 1024 K for this element format and accumulation mode, in µs.
double mx_split_tile_us(int elem, bool exact);

}  // namespace nvfp4
