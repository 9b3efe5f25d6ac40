// C ABI of the NVFP4 library (declared in include/nvfp4.h): host-side argument
// validation, then dispatch to the kernel launchers.  No entry point allocates
// memory or keeps state; every error is reported before anything is enqueued.
#include "nvfp4.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

using namespace nvfp4;

// Scratch of nvfp4_quantize_noalloc: the amax pass's per-workgroup partial
// maxima (at most kMaxPartials floats for a tensor of any size, 2 KiB).  Each
// device the library runs on holds its own copy until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: kernels
// get the device address that hipGetSymbolAddress returns for the device.
static __device__ __align__(256) float scratch[kMaxPartials];

namespace {

constexpr int64_t kMaxGridY = 65535;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dtype_size(int dt) { return dt == NVFP4_BF16 ? 2 : 4; }

bool valid_dtype(int dt) { return dt == NVFP4_F32 || dt == NVFP4_BF16; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The output tensor a layout implies for an input of rows x cols.
nvfp4_status check_out(const nvfp4_tensor* t, int64_t r, int64_t c, int mode) {
    if (!t->tensor_scale) return NVFP4_ERR_NULL;
    if (r > 0 && c > 0 && (!t->codes || !t->scales)) return NVFP4_ERR_NULL;
    if (t->rows != r || t->cols != c || t->scale_mode != mode) return NVFP4_ERR_SHAPE;
    if (!aligned(t->codes, 16)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// A GEMM operand: shape, scale layout, pointers, alignment.
nvfp4_status check_operand(const nvfp4_tensor* t) {
    if (!t) return NVFP4_ERR_NULL;
    if (t->rows < 0 || t->cols < 0) return NVFP4_ERR_SHAPE;
    if (t->scale_mode != NVFP4_SCALE_1D && t->scale_mode != NVFP4_SCALE_2D) return NVFP4_ERR_ENUM;
    if (t->cols % 16) return NVFP4_ERR_SHAPE;
    if (t->scale_mode == NVFP4_SCALE_2D && t->rows % 16) return NVFP4_ERR_SHAPE;
    if (t->rows > 0 && t->cols > 0 && (!t->codes || !t->scales)) return NVFP4_ERR_NULL;
    if (!t->tensor_scale) return NVFP4_ERR_NULL;
    if (!aligned(t->codes, 16)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

Operand as_operand(const nvfp4_tensor* t) {
    return Operand{t->codes, t->scales, t->tensor_scale, t->scale_mode == NVFP4_SCALE_2D ? 1 : 0};
}

}  // namespace

extern "C" {

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols, const nvfp4_quant_opts* opts) {
    (void)rows;
    (void)cols;
    if (opts && opts->amax_in) return 0;
    return kQuantWorkspaceBytes;
}

}  // extern "C"

namespace {

// Argument checks of nvfp4_quantize other than the workspace; NVFP4_OK when
// the request can be launched.
nvfp4_status check_quantize(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols, int64_t ld,
                            const nvfp4_quant_opts* opts, nvfp4_tensor* out) {
    if (!opts || !out) return NVFP4_ERR_NULL;
    if (!valid_dtype(dt)) return NVFP4_ERR_ENUM;
    const int layout = opts->layout;
    if (layout < NVFP4_ROW_1D || layout > NVFP4_BLK_2D) return NVFP4_ERR_ENUM;
    if (opts->round != NVFP4_RNE && opts->round != NVFP4_SR) return NVFP4_ERR_ENUM;
    if (rows < 0 || cols < 0 || ld < cols) return NVFP4_ERR_SHAPE;
    const bool row_blocks = layout == NVFP4_ROW_1D || layout == NVFP4_ROW_COL_1D || layout == NVFP4_BLK_2D;
    const bool col_blocks = layout == NVFP4_COL_1D || layout == NVFP4_ROW_COL_1D || layout == NVFP4_BLK_2D;
    if (row_blocks && cols % 16) return NVFP4_ERR_SHAPE;
    if (col_blocks && rows % 16) return NVFP4_ERR_SHAPE;
    if (opts->hadamard && layout == NVFP4_BLK_2D) return NVFP4_ERR_UNSUPPORTED;
    const bool empty = rows == 0 || cols == 0;
    if (!empty && !x) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || (ld * (int64_t)dtype_size(dt)) % 16) return NVFP4_ERR_ALIGN;

    nvfp4_status st;
    switch (layout) {
        case NVFP4_ROW_1D: st = check_out(&out[0], rows, cols, NVFP4_SCALE_1D); break;
        case NVFP4_COL_1D: st = check_out(&out[0], cols, rows, NVFP4_SCALE_1D); break;
        case NVFP4_BLK_2D: st = check_out(&out[0], rows, cols, NVFP4_SCALE_2D); break;
        default:
            st = check_out(&out[0], rows, cols, NVFP4_SCALE_1D);
            if (st == NVFP4_OK) st = check_out(&out[1], cols, rows, NVFP4_SCALE_1D);
    }
    if (st != NVFP4_OK) return st;

    // grid-size limits of the launches (y counts row tiles / row bands)
    if (cdiv(cols, 128) > 0x7FFFFFFF) return NVFP4_ERR_UNSUPPORTED;
    if ((layout == NVFP4_COL_1D || layout == NVFP4_ROW_COL_1D) && cdiv(rows, 256) > kMaxGridY)
        return NVFP4_ERR_UNSUPPORTED;
    if (layout == NVFP4_BLK_2D && cdiv(rows, 64) > kMaxGridY) return NVFP4_ERR_UNSUPPORTED;
    return NVFP4_OK;
}

nvfp4_status launch_checked_quantize(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols,
                                     int64_t ld, const nvfp4_quant_opts* opts, nvfp4_tensor* out,
                                     float* ws, void* stream) {
    const int layout = opts->layout;
    QOut o[2];
    o[0] = QOut{out[0].codes, out[0].scales, out[0].tensor_scale};
    if (layout == NVFP4_ROW_COL_1D) o[1] = QOut{out[1].codes, out[1].scales, out[1].tensor_scale};
    else o[1] = QOut{nullptr, nullptr, nullptr};
    hipError_t e = launch_quantize(x, dt == NVFP4_BF16, rows, cols, ld, layout, opts->round == NVFP4_SR,
                                   opts->sr_seed, opts->hadamard != 0, opts->hadamard_seed,
                                   opts->amax_in, opts->amax_out, o, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device `stream` belongs to, looked up
// once per device with that device current; NULL on failure.
float* scratch_on_device_of(hipStream_t stream) {
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols, int64_t ld,
                            const nvfp4_quant_opts* opts, nvfp4_tensor* out, void* ws,
                            size_t ws_bytes, void* stream) {
    nvfp4_status st = check_quantize(x, dt, rows, cols, ld, opts, out);
    if (st != NVFP4_OK) return st;
    if (rows > 0 && cols > 0 && !opts->amax_in) {
        if (!ws) return NVFP4_ERR_WORKSPACE;
        if (ws_bytes < kQuantWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    }
    return launch_checked_quantize(x, dt, rows, cols, ld, opts, out, static_cast<float*>(ws), stream);
}

nvfp4_status nvfp4_quantize_noalloc(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols, int64_t ld,
                                    const nvfp4_quant_opts* opts, nvfp4_tensor* out, void* stream) {
    nvfp4_status st = check_quantize(x, dt, rows, cols, ld, opts, out);
    if (st != NVFP4_OK) return st;
    // the amax pass writes at most kMaxPartials partials whatever the size, so
    // no request needs more scratch than the array holds
    static_assert(sizeof(scratch) >= kQuantWorkspaceBytes, "scratch smaller than the quantize workspace");
    float* ws = nullptr;
    if (rows > 0 && cols > 0 && !opts->amax_in) {
        ws = scratch_on_device_of(static_cast<hipStream_t>(stream));
        if (!ws) return NVFP4_ERR_HIP;
    }
    return launch_checked_quantize(x, dt, rows, cols, ld, opts, out, ws, stream);
}

nvfp4_status nvfp4_requantize(const nvfp4_tensor* in, const nvfp4_quant_opts* opts, nvfp4_tensor* out,
                              void* ws, size_t ws_bytes, void* stream) {
    if (!in || !opts || !out) return NVFP4_ERR_NULL;
    if (opts->layout < NVFP4_ROW_1D || opts->layout > NVFP4_BLK_2D) return NVFP4_ERR_ENUM;
    if (opts->round != NVFP4_RNE && opts->round != NVFP4_SR) return NVFP4_ERR_ENUM;
    nvfp4_status st = check_operand(in);
    if (st != NVFP4_OK) return st;
    if (in->scale_mode != NVFP4_SCALE_1D) return NVFP4_ERR_UNSUPPORTED;
    if (opts->layout != NVFP4_COL_1D) return NVFP4_ERR_UNSUPPORTED;
    const int64_t rows = in->rows, cols = in->cols;
    if (rows % 16) return NVFP4_ERR_SHAPE;
    st = check_out(out, cols, rows, NVFP4_SCALE_1D);
    if (st != NVFP4_OK) return st;
    if (cdiv(rows, 256) > kMaxGridY) return NVFP4_ERR_UNSUPPORTED;
    const bool empty = rows == 0 || cols == 0;
    if (!empty && !opts->amax_in) {
        if (!ws) return NVFP4_ERR_WORKSPACE;
        if (ws_bytes < kQuantWorkspaceBytes) return NVFP4_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    }
    const QOut o{out->codes, out->scales, out->tensor_scale};
    hipError_t e = launch_requantize(in->codes, in->scales, in->tensor_scale, rows, cols,
                                     opts->round == NVFP4_SR, opts->sr_seed, opts->hadamard != 0,
                                     opts->hadamard_seed, opts->amax_in, opts->amax_out, &o,
                                     static_cast<float*>(ws), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_dequantize(const nvfp4_tensor* q, void* y, int32_t dt /* nvfp4_dtype */, int64_t ld,
                              void* stream) {
    if (!q) return NVFP4_ERR_NULL;
    if (!valid_dtype(dt)) return NVFP4_ERR_ENUM;
    nvfp4_status st = check_operand(q);
    if (st != NVFP4_OK) return st;
    if (ld < q->cols) return NVFP4_ERR_SHAPE;
    const bool empty = q->rows == 0 || q->cols == 0;
    if (!empty && !y) return NVFP4_ERR_NULL;
    if (!aligned(y, 16) || (ld * (int64_t)dtype_size(dt)) % 16) return NVFP4_ERR_ALIGN;
    hipError_t e = launch_dequantize(q->codes, q->scales, q->tensor_scale, q->rows, q->cols,
                                     q->scale_mode == NVFP4_SCALE_2D, y, dt == NVFP4_BF16, ld,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

size_t nvfp4_gemm_workspace_size(const nvfp4_tensor* A, const nvfp4_tensor* B, int32_t c_dt /* nvfp4_dtype */,
                                 int32_t ep /* nvfp4_epilogue */) {
    if (!A || !B || !valid_dtype(c_dt) || ep != NVFP4_EPI_NONE) return 0;
    if (A->rows < 0 || B->rows < 0 || A->cols != B->cols) return 0;
    int cus = 0;
    if (device_cus(cus) != hipSuccess) return 0;
    const GemmSplit sp = gemm_split_plan(A->rows, B->rows, A->cols, false, cus);
    return sp.split > 1 ? (size_t)sp.bytes : 0;
}

nvfp4_status nvfp4_gemm(const nvfp4_tensor* A, const nvfp4_tensor* B, void* C, int32_t c_dt /* nvfp4_dtype */,
                        int64_t ldc, int32_t ep /* nvfp4_epilogue */, void* ws, size_t ws_bytes, void* stream) {
    if (!A || !B) return NVFP4_ERR_NULL;
    if (!valid_dtype(c_dt)) return NVFP4_ERR_ENUM;
    if (ep != NVFP4_EPI_NONE && ep != NVFP4_EPI_SWIGLU) return NVFP4_ERR_ENUM;
    nvfp4_status st = check_operand(A);
    if (st != NVFP4_OK) return st;
    st = check_operand(B);
    if (st != NVFP4_OK) return st;
    if (A->cols != B->cols) return NVFP4_ERR_SHAPE;
    const int64_t M = A->rows, N = B->rows, K = A->cols;
    const bool swiglu = ep == NVFP4_EPI_SWIGLU;
    if (swiglu) {
        if (N % 2 || (N / 2) % 16) return NVFP4_ERR_SHAPE;
        if (c_dt != NVFP4_BF16) return NVFP4_ERR_UNSUPPORTED;
    }
    const int64_t ncols = swiglu ? N / 2 : N;
    if (ldc < ncols) return NVFP4_ERR_SHAPE;
    if (M > 0 && ncols > 0 && !C) return NVFP4_ERR_NULL;
    if (!aligned(C, dtype_size(c_dt))) return NVFP4_ERR_ALIGN;
    if (cdiv(M, 128) > kMaxGridY) return NVFP4_ERR_UNSUPPORTED;
    if (ws && !aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    hipError_t e = launch_gemm(as_operand(A), as_operand(B), M, N, K, C, c_dt == NVFP4_BF16, ldc, swiglu,
                               ws, ws ? ws_bytes : 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_grouped_gemm(int32_t G, const nvfp4_tensor* A, const int64_t* offsets,
                                const nvfp4_tensor* B, void* C, int32_t c_dt /* nvfp4_dtype */, int64_t ldc,
                                int32_t ep /* nvfp4_epilogue */, float* amax_out, void* ws, size_t ws_bytes,
                                void* stream) {
    (void)ws;
    (void)ws_bytes;
    if (!A || !B || !offsets) return NVFP4_ERR_NULL;
    if (!valid_dtype(c_dt)) return NVFP4_ERR_ENUM;
    if (ep != NVFP4_EPI_NONE && ep != NVFP4_EPI_SWIGLU) return NVFP4_ERR_ENUM;
    if (G < 1) return NVFP4_ERR_SHAPE;
    nvfp4_status st = check_operand(A);
    if (st != NVFP4_OK) return st;
    st = check_operand(B);
    if (st != NVFP4_OK) return st;
    if (A->scale_mode != NVFP4_SCALE_1D) return NVFP4_ERR_UNSUPPORTED;
    if (A->cols != B->cols) return NVFP4_ERR_SHAPE;
    if (B->rows % G) return NVFP4_ERR_SHAPE;
    const int64_t Ng = B->rows / G, K = A->cols, total = A->rows;
    if (B->scale_mode == NVFP4_SCALE_2D && Ng % 16) return NVFP4_ERR_SHAPE;
    const bool swiglu = ep == NVFP4_EPI_SWIGLU;
    if (swiglu) {
        if (Ng % 2 || (Ng / 2) % 16) return NVFP4_ERR_SHAPE;
        if (c_dt != NVFP4_BF16) return NVFP4_ERR_UNSUPPORTED;
    } else if (amax_out) {
        return NVFP4_ERR_UNSUPPORTED;
    }
    const int64_t ncols = swiglu ? Ng / 2 : Ng;
    if (ldc < ncols) return NVFP4_ERR_SHAPE;
    if (total > 0 && ncols > 0 && !C) return NVFP4_ERR_NULL;
    if (!aligned(C, dtype_size(c_dt))) return NVFP4_ERR_ALIGN;
    if (cdiv(total, 128) + G > kMaxGridY) return NVFP4_ERR_UNSUPPORTED;
    hipError_t e = launch_grouped_gemm(G, as_operand(A), offsets, total, as_operand(B), Ng, K, C,
                                       c_dt == NVFP4_BF16, ldc, swiglu, amax_out,
                                       static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// ---------------------------------------------------------------- MX formats
nvfp4_status nvfp4_mx_quantize(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols, int64_t ld,
                               int32_t layout /* nvfp4_layout */, int32_t round /* nvfp4_round */, uint64_t sr_seed,
                               nvfp4_mx_tensor* out, void* stream) {
    if (!out) return NVFP4_ERR_NULL;
    if (!valid_dtype(dt)) return NVFP4_ERR_ENUM;
    if (layout < NVFP4_ROW_1D || layout > NVFP4_BLK_2D) return NVFP4_ERR_ENUM;
    if (round != NVFP4_RNE && round != NVFP4_SR) return NVFP4_ERR_ENUM;
    if (out->elem != NVFP4_MX_E4M3 && out->elem != NVFP4_MX_E2M1) return NVFP4_ERR_ENUM;
    if (layout != NVFP4_ROW_1D && layout != NVFP4_COL_1D) return NVFP4_ERR_UNSUPPORTED;
    if (rows < 0 || cols < 0 || ld < cols) return NVFP4_ERR_SHAPE;
    const bool col = layout == NVFP4_COL_1D;
    if ((col ? rows : cols) % 32) return NVFP4_ERR_SHAPE;
    const int64_t orows = col ? cols : rows, ocols = col ? rows : cols;
    if (out->rows != orows || out->cols != ocols) return NVFP4_ERR_SHAPE;
    const bool empty = rows == 0 || cols == 0;
    if (!empty && (!x || !out->codes || !out->scales)) return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || (ld * (int64_t)dtype_size(dt)) % 16 || !aligned(out->codes, 16))
        return NVFP4_ERR_ALIGN;
    if (col ? cdiv(rows, 256) > kMaxGridY : cdiv(cols, 512) > 0x7FFFFFFF) return NVFP4_ERR_UNSUPPORTED;
    hipError_t e = launch_mx_quantize(x, dt == NVFP4_BF16, rows, cols, ld, col ? kLayoutCol : kLayoutRow,
                                      out->elem == NVFP4_MX_E4M3 ? kMxE4M3 : kMxE2M1, round == NVFP4_SR,
                                      sr_seed, out->codes, out->scales, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

nvfp4_status nvfp4_mx_dequantize(const nvfp4_mx_tensor* q, void* y, int32_t dt /* nvfp4_dtype */, int64_t ld,
                                 void* stream) {
    if (!q) return NVFP4_ERR_NULL;
    if (!valid_dtype(dt)) return NVFP4_ERR_ENUM;
    if (q->elem != NVFP4_MX_E4M3 && q->elem != NVFP4_MX_E2M1) return NVFP4_ERR_ENUM;
    if (q->rows < 0 || q->cols < 0 || q->cols % 32 || ld < q->cols) return NVFP4_ERR_SHAPE;
    const bool empty = q->rows == 0 || q->cols == 0;
    if (!empty && (!y || !q->codes || !q->scales)) return NVFP4_ERR_NULL;
    if (!aligned(y, 16) || (ld * (int64_t)dtype_size(dt)) % 16 || !aligned(q->codes, 16))
        return NVFP4_ERR_ALIGN;
    if (cdiv(q->cols / 8, 64) > 0x7FFFFFFF) return NVFP4_ERR_UNSUPPORTED;
    hipError_t e = launch_mx_dequantize(q->codes, q->scales, q->elem == NVFP4_MX_E4M3 ? kMxE4M3 : kMxE2M1,
                                        q->rows, q->cols, y, dt == NVFP4_BF16, ld,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

size_t nvfp4_mx_gemm_workspace_size(const nvfp4_mx_tensor* A, const nvfp4_mx_tensor* B, int32_t c_dt /* nvfp4_dtype */,
                                    int32_t accum) {
    if (!A || !B || !valid_dtype(c_dt)) return 0;
    if (accum != NVFP4_MX_ACC_NATIVE && accum != NVFP4_MX_ACC_EXACT) return 0;
    if (A->rows < 0 || B->rows < 0 || A->cols != B->cols) return 0;
    int cus = 0;
    if (device_cus(cus) != hipSuccess) return 0;
    const GemmSplit sp =
        mx_gemm_split_plan(A->rows, B->rows, A->cols, mx_split_tile_us(A->elem == NVFP4_MX_E4M3 ? kMxE4M3 : kMxE2M1, accum == NVFP4_MX_ACC_EXACT), cus);
    return sp.split > 1 ? (size_t)sp.bytes : 0;
}

nvfp4_status nvfp4_mx_gemm(const nvfp4_mx_tensor* A, const nvfp4_mx_tensor* B, void* C, int32_t c_dt /* nvfp4_dtype */,
                           int64_t ldc, int32_t accum, void* ws, size_t ws_bytes, void* stream) {
    if (!A || !B) return NVFP4_ERR_NULL;
    if (!valid_dtype(c_dt)) return NVFP4_ERR_ENUM;
    if (accum != NVFP4_MX_ACC_NATIVE && accum != NVFP4_MX_ACC_EXACT) return NVFP4_ERR_ENUM;
    for (const nvfp4_mx_tensor* t : {A, B}) {
        if (t->elem != NVFP4_MX_E4M3 && t->elem != NVFP4_MX_E2M1) return NVFP4_ERR_ENUM;
        if (t->rows < 0 || t->cols < 0 || t->cols % 32) return NVFP4_ERR_SHAPE;
    }
    if (A->cols != B->cols) return NVFP4_ERR_SHAPE;
    if (A->elem != B->elem) return NVFP4_ERR_UNSUPPORTED;
    const int64_t M = A->rows, N = B->rows, K = A->cols;
    if (K % 64) return NVFP4_ERR_UNSUPPORTED;
    // the kernels keep per-lane byte offsets inside a 256-row tile in 32 bits
    const uint64_t row_bytes = (uint64_t)(A->elem == NVFP4_MX_E4M3 ? K : K / 2);
    if (256 * row_bytes >= ((uint64_t)1 << 32)) return NVFP4_ERR_UNSUPPORTED;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    if (M > 0 && N > 0) {
        if (!C) return NVFP4_ERR_NULL;
        if (K > 0 && (!A->codes || !A->scales || !B->codes || !B->scales)) return NVFP4_ERR_NULL;
    }
    if (!aligned(C, dtype_size(c_dt)) || !aligned(A->codes, 16) || !aligned(B->codes, 16) ||
        !aligned(A->scales, 2) || !aligned(B->scales, 2))
        return NVFP4_ERR_ALIGN;
    if (cdiv(M, 256) > kMaxGridY) return NVFP4_ERR_UNSUPPORTED;
    if (ws && !aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    hipError_t e = launch_mx_gemm(A->codes, A->scales, B->codes, B->scales,
                                  A->elem == NVFP4_MX_E4M3 ? kMxE4M3 : kMxE2M1, M, N, K, C, c_dt == NVFP4_BF16,
                                  ldc, accum == NVFP4_MX_ACC_EXACT, ws, ws ? ws_bytes : 0,
                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

const char* nvfp4_status_string(int32_t s /* nvfp4_status */) {
    switch (s) {
        case NVFP4_OK: return "ok";
        case NVFP4_ERR_NULL: return "a required pointer is NULL";
        case NVFP4_ERR_ENUM: return "an enum argument is out of range";
        case NVFP4_ERR_SHAPE: return "invalid or inconsistent shape";
        case NVFP4_ERR_ALIGN: return "pointer or leading dimension misaligned";
        case NVFP4_ERR_UNSUPPORTED: return "unsupported combination";
        case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
        case NVFP4_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

int32_t nvfp4_version(void) { return 100; }

}  // extern "C"
