/* Host-side argument validation of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure only):
 * tests/test_abi_sanitize.py builds the ABI layer (csrc/nvfp4_api.hip) with
 * the sanitizers on its host code, links it with the library's kernel
 * objects, builds this C driver against it with the same sanitizers, and
 * runs it.  Every call below passes an argument that validation must refuse
 * (the expected status is stated with it), so nothing is ever launched:
 * pointers that are only checked for alignment and never dereferenced are
 * plain integers here, and enumerated arguments take out-of-range integers
 * as a C caller may pass them.  Prints "ok" at the end; a wrong status or a
 * sanitizer report fails.
 */
#include <stdint.h>
#include <stdio.h>

#include "nvfp4.h"

static int failures = 0;

#define CHECK(expr, want)                                                                     \
    do {                                                                                      \
        const int got_ = (int)(expr);                                                         \
        if (got_ != (int)(want)) {                                                            \
            fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_,  \
                    (int)(want));                                                             \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

#define X ((const void*)(uintptr_t)65536) /* an aligned input address, never read */
#define Y ((void*)(uintptr_t)65536)       /* an aligned output address, never written */
#define WS ((void*)(uintptr_t)65536)

static nvfp4_tensor T(int64_t rows, int64_t cols, int mode, uintptr_t codes) {
    nvfp4_tensor t;
    t.codes = (uint8_t*)codes;
    t.scales = (uint8_t*)(uintptr_t)8192;
    t.tensor_scale = (float*)(uintptr_t)12288;
    t.rows = rows;
    t.cols = cols;
    t.scale_mode = mode;
    return t;
}

static nvfp4_quant_opts O(int layout, int round, int had) {
    nvfp4_quant_opts o;
    o.layout = layout;
    o.round = round;
    o.sr_seed = 1;
    o.hadamard = had;
    o.hadamard_seed = 2;
    o.amax_in = NULL;
    o.amax_out = NULL;
    return o;
}

/* nvfp4_quantize with its outputs and workspace given by value */
static nvfp4_status quant(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld, nvfp4_quant_opts o,
                          nvfp4_tensor t0, nvfp4_tensor t1, void* ws, size_t ws_bytes) {
    nvfp4_tensor outs[2];
    outs[0] = t0;
    outs[1] = t1;
    return nvfp4_quantize(x, (nvfp4_dtype)dt, rows, cols, ld, &o, outs, ws, ws_bytes, NULL);
}

static void quantize_cases(void) {
    const nvfp4_tensor ok = T(32, 32, 0, 4096), none = T(0, 0, 0, 4096);
    const nvfp4_quant_opts row = O(0, 0, 0);
    const size_t W = 1 << 20;
    CHECK(quant(NULL, 1, 32, 32, 32, row, ok, none, WS, W), NVFP4_ERR_NULL);
    CHECK(quant(X, 7, 32, 32, 32, row, ok, none, WS, W), NVFP4_ERR_ENUM);
    CHECK(quant(X, -1, 32, 32, 32, row, ok, none, WS, W), NVFP4_ERR_ENUM);
    CHECK(quant(X, 1, 32, 32, 32, O(9, 0, 0), ok, none, WS, W), NVFP4_ERR_ENUM);
    CHECK(quant(X, 1, 32, 32, 32, O(-2, 0, 0), ok, none, WS, W), NVFP4_ERR_ENUM);
    CHECK(quant(X, 1, 32, 32, 32, O(0, 5, 0), ok, none, WS, W), NVFP4_ERR_ENUM);
    CHECK(quant(X, 1, 32, 24, 32, row, T(32, 24, 0, 4096), none, WS, W), NVFP4_ERR_SHAPE);    /* cols % 16 */
    CHECK(quant(X, 1, 24, 32, 32, O(1, 0, 0), T(32, 24, 0, 4096), none, WS, W), NVFP4_ERR_SHAPE); /* rows % 16 */
    CHECK(quant(X, 1, 32, 32, 16, row, ok, none, WS, W), NVFP4_ERR_SHAPE);                   /* ld < cols */
    CHECK(quant(X, 1, -16, 32, 32, row, ok, none, WS, W), NVFP4_ERR_SHAPE);
    CHECK(quant(X, 1, 32, 32, 36, row, ok, none, WS, W), NVFP4_ERR_ALIGN);                   /* 72-byte rows */
    CHECK(quant((const void*)(uintptr_t)65538, 1, 32, 32, 32, row, ok, none, WS, W), NVFP4_ERR_ALIGN);
    CHECK(quant(X, 1, 32, 32, 32, O(3, 0, 1), T(32, 32, 1, 4096), none, WS, W), NVFP4_ERR_UNSUPPORTED);
    CHECK(quant(X, 1, 32, 32, 32, O(2, 0, 1), ok, T(16, 32, 0, 4096), WS, W), NVFP4_ERR_SHAPE);
    CHECK(quant(X, 1, 32, 32, 32, row, T(32, 32, 1, 4096), none, WS, W), NVFP4_ERR_SHAPE);    /* scale mode */
    CHECK(quant(X, 1, 32, 32, 32, O(1, 0, 0), T(32, 64, 0, 4096), none, WS, W), NVFP4_ERR_SHAPE);
    CHECK(quant(X, 1, 32, 32, 32, row, T(32, 32, 0, 0), none, WS, W), NVFP4_ERR_NULL);
    CHECK(quant(X, 1, 32, 32, 32, row, T(32, 32, 0, 4100), none, WS, W), NVFP4_ERR_ALIGN);
    CHECK(quant(X, 1, 32, 32, 32, row, ok, none, NULL, W), NVFP4_ERR_WORKSPACE);
    CHECK(quant(X, 1, 32, 32, 32, row, ok, none, WS, 16), NVFP4_ERR_WORKSPACE);
    nvfp4_tensor outs[2];
    outs[0] = ok;
    outs[1] = none;
    CHECK(nvfp4_quantize(X, NVFP4_BF16, 32, 32, 32, NULL, outs, WS, W, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_quantize(X, NVFP4_BF16, 32, 32, 32, &row, NULL, WS, W, NULL), NVFP4_ERR_NULL);
    /* the allocation-free variant validates the same way */
    CHECK(nvfp4_quantize_noalloc(X, NVFP4_BF16, 32, 32, 32, NULL, NULL, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_quantize_noalloc(NULL, NVFP4_BF16, 32, 32, 32, &row, outs, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_quantize_noalloc(X, (nvfp4_dtype)5, 32, 32, 32, &row, outs, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_quantize_noalloc(X, NVFP4_BF16, 32, 32, 36, &row, outs, NULL), NVFP4_ERR_ALIGN);
    /* the workspace size is a pure host computation */
    CHECK(nvfp4_quantize_workspace_size(32, 32, &row) > 0, 1);
    CHECK(nvfp4_quantize_workspace_size(32, 32, NULL) > 0, 1);
}

static void dequantize_cases(void) {
    const nvfp4_tensor q = T(32, 32, 0, 4096), bad = T(32, 24, 0, 4096), bad2 = T(24, 32, 1, 4096);
    CHECK(nvfp4_dequantize(NULL, Y, NVFP4_F32, 32, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_dequantize(&q, NULL, NVFP4_F32, 32, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_dequantize(&q, Y, (nvfp4_dtype)3, 32, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_dequantize(&q, Y, NVFP4_F32, 16, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_dequantize(&q, (void*)(uintptr_t)65540, NVFP4_F32, 32, NULL), NVFP4_ERR_ALIGN);
    CHECK(nvfp4_dequantize(&bad, Y, NVFP4_F32, 32, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_dequantize(&bad2, Y, NVFP4_F32, 32, NULL), NVFP4_ERR_SHAPE);
}

static void requantize_cases(void) {
    const nvfp4_tensor q = T(64, 32, 0, 4096), q2d = T(64, 32, 1, 4096), q40 = T(40, 32, 0, 4096);
    nvfp4_tensor out = T(32, 64, 0, 4096), out40 = T(32, 40, 0, 4096), wrong = T(64, 32, 0, 4096),
                 misaligned = T(32, 64, 0, 4100);
    const nvfp4_quant_opts col = O(1, 0, 0), bad_layout = O(7, 0, 0), bad_round = O(1, 5, 0), row = O(0, 0, 0);
    const size_t W = 1 << 20;
    CHECK(nvfp4_requantize(NULL, &col, &out, WS, W, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_requantize(&q, &bad_layout, &out, WS, W, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_requantize(&q, &bad_round, &out, WS, W, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_requantize(&q, &row, &out, WS, W, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_requantize(&q2d, &col, &out, WS, W, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_requantize(&q40, &col, &out40, WS, W, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_requantize(&q, &col, &wrong, WS, W, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_requantize(&q, &col, &misaligned, WS, W, NULL), NVFP4_ERR_ALIGN);
    CHECK(nvfp4_requantize(&q, &col, &out, NULL, W, NULL), NVFP4_ERR_WORKSPACE);
    CHECK(nvfp4_requantize(&q, &col, &out, WS, 16, NULL), NVFP4_ERR_WORKSPACE);
}

static void gemm_cases(void) {
    const nvfp4_tensor a = T(64, 64, 0, 4096), b = T(32, 64, 0, 4096), b48 = T(48, 64, 0, 4096),
                       b2 = T(32, 48, 0, 4096), a3 = T(64, 40, 0, 4096), b3 = T(32, 40, 0, 4096);
    CHECK(nvfp4_gemm(NULL, &b, Y, NVFP4_F32, 32, NVFP4_EPI_NONE, NULL, 0, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_gemm(&a, &b, Y, (nvfp4_dtype)9, 32, NVFP4_EPI_NONE, NULL, 0, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_gemm(&a, &b, Y, NVFP4_F32, 32, (nvfp4_epilogue)4, NULL, 0, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_gemm(&a, &b, Y, NVFP4_F32, 32, NVFP4_EPI_SWIGLU, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_gemm(&a, &b, Y, NVFP4_BF16, 15, NVFP4_EPI_SWIGLU, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_gemm(&a, &b48, Y, NVFP4_BF16, 24, NVFP4_EPI_SWIGLU, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_gemm(&a, &b2, Y, NVFP4_F32, 32, NVFP4_EPI_NONE, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_gemm(&a, &b, Y, NVFP4_F32, 16, NVFP4_EPI_NONE, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_gemm(&a, &b, NULL, NVFP4_F32, 32, NVFP4_EPI_NONE, NULL, 0, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_gemm(&a3, &b3, Y, NVFP4_F32, 32, NVFP4_EPI_NONE, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    /* grouped */
    const nvfp4_tensor ga = T(100, 64, 0, 4096), gb = T(4 * 32, 64, 1, 4096);
    const int64_t* off = (const int64_t*)(uintptr_t)65536;
    float* amax = (float*)(uintptr_t)65536;
    CHECK(nvfp4_grouped_gemm(4, &ga, NULL, &gb, Y, NVFP4_BF16, 32, NVFP4_EPI_NONE, NULL, NULL, 0, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_grouped_gemm(0, &ga, off, &gb, Y, NVFP4_BF16, 32, NVFP4_EPI_NONE, NULL, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_grouped_gemm(3, &ga, off, &gb, Y, NVFP4_BF16, 32, NVFP4_EPI_NONE, NULL, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_grouped_gemm(4, &ga, off, &gb, Y, NVFP4_F32, 16, NVFP4_EPI_SWIGLU, NULL, NULL, 0, NULL),
          NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_grouped_gemm(4, &ga, off, &gb, Y, NVFP4_BF16, 8, NVFP4_EPI_SWIGLU, NULL, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_grouped_gemm(4, &ga, off, &gb, Y, NVFP4_BF16, 32, NVFP4_EPI_NONE, amax, NULL, 0, NULL),
          NVFP4_ERR_UNSUPPORTED);
}

static nvfp4_mx_tensor MX(int64_t rows, int64_t cols, int elem, uintptr_t codes, uintptr_t scales) {
    nvfp4_mx_tensor t;
    t.codes = (uint8_t*)codes;
    t.scales = (uint8_t*)scales;
    t.rows = rows;
    t.cols = cols;
    t.elem = elem;
    return t;
}

static void mx_cases(void) {
    nvfp4_mx_tensor t = MX(64, 64, 0, 4096, 8192), t48 = MX(64, 48, 0, 4096, 8192), t96 = MX(64, 96, 0, 4096, 8192),
                    tbad = MX(64, 64, 2, 4096, 8192), tmis = MX(64, 64, 0, 4104, 8192);
    const nvfp4_dtype bf = NVFP4_BF16;
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 64, NVFP4_ROW_1D, NVFP4_RNE, 1, NULL, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_mx_quantize(NULL, bf, 64, 64, 64, NVFP4_ROW_1D, NVFP4_RNE, 1, &t, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_mx_quantize(X, (nvfp4_dtype)3, 64, 64, 64, NVFP4_ROW_1D, NVFP4_RNE, 1, &t, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 64, (nvfp4_layout)7, NVFP4_RNE, 1, &t, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 64, NVFP4_ROW_1D, (nvfp4_round)2, 1, &t, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 64, NVFP4_ROW_1D, NVFP4_RNE, 1, &tbad, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 64, NVFP4_ROW_COL_1D, NVFP4_RNE, 1, &t, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 64, NVFP4_BLK_2D, NVFP4_RNE, 1, &t, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 48, 48, NVFP4_ROW_1D, NVFP4_RNE, 1, &t48, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_quantize(X, bf, 48, 64, 64, NVFP4_COL_1D, NVFP4_RNE, 1, &t48, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 96, 96, NVFP4_COL_1D, NVFP4_RNE, 1, &t96, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 32, NVFP4_ROW_1D, NVFP4_RNE, 1, &t, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 68, NVFP4_ROW_1D, NVFP4_RNE, 1, &t, NULL), NVFP4_ERR_ALIGN);
    CHECK(nvfp4_mx_quantize(X, bf, 64, 64, 64, NVFP4_ROW_1D, NVFP4_RNE, 1, &tmis, NULL), NVFP4_ERR_ALIGN);
    /* dequantize */
    nvfp4_mx_tensor e5 = MX(64, 64, 5, 4096, 8192);
    CHECK(nvfp4_mx_dequantize(NULL, Y, NVFP4_F32, 64, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_mx_dequantize(&e5, Y, NVFP4_F32, 64, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_dequantize(&t, Y, (nvfp4_dtype)9, 64, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_dequantize(&t48, Y, NVFP4_F32, 48, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_dequantize(&t, Y, NVFP4_F32, 32, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_dequantize(&t, NULL, NVFP4_F32, 64, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_mx_dequantize(&t, (void*)(uintptr_t)65540, NVFP4_F32, 64, NULL), NVFP4_ERR_ALIGN);
    CHECK(nvfp4_mx_dequantize(&t, Y, NVFP4_F32, 66, NULL), NVFP4_ERR_ALIGN);
    /* GEMM */
    nvfp4_mx_tensor a = MX(64, 128, 0, 4096, 8192), b = MX(32, 128, 0, 4096, 8192), a96 = MX(64, 96, 0, 4096, 8192),
                    b96 = MX(32, 96, 0, 4096, 8192), a80 = MX(64, 80, 0, 4096, 8192), b80 = MX(32, 80, 0, 4096, 8192),
                    b192 = MX(32, 192, 0, 4096, 8192), bfp4 = MX(32, 128, 1, 4096, 8192),
                    a3 = MX(64, 128, 3, 4096, 8192), amis = MX(64, 128, 0, 4100, 8192),
                    asmis = MX(64, 128, 0, 4096, 8193), aneg = MX(-1, 128, 0, 4096, 8192);
    const nvfp4_dtype f32 = NVFP4_F32;
    const nvfp4_mx_accum nat = NVFP4_MX_ACC_NATIVE;
    CHECK(nvfp4_mx_gemm(NULL, NULL, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_mx_gemm(&a, &b, Y, (nvfp4_dtype)4, 32, nat, NULL, 0, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_gemm(&a, &b, Y, f32, 32, (nvfp4_mx_accum)2, NULL, 0, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_gemm(&a, &b, Y, f32, 32, (nvfp4_mx_accum)-1, NULL, 0, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_gemm(&a3, &b, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_ENUM);
    CHECK(nvfp4_mx_gemm(&a96, &b96, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_mx_gemm(&a80, &b80, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_gemm(&a, &b192, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_gemm(&a, &bfp4, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_mx_gemm(&a, &b, Y, f32, 16, nat, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    CHECK(nvfp4_mx_gemm(&a, &b, NULL, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_NULL);
    CHECK(nvfp4_mx_gemm(&a, &b, (void*)(uintptr_t)65538, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_ALIGN);
    CHECK(nvfp4_mx_gemm(&amis, &b, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_ALIGN);
    CHECK(nvfp4_mx_gemm(&asmis, &b, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_ALIGN);
    CHECK(nvfp4_mx_gemm(&aneg, &b, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_SHAPE);
    const int64_t K4 = (int64_t)1 << 24;
    nvfp4_mx_tensor ak = MX(64, K4, 0, 4096, 8192), bk = MX(32, K4, 0, 4096, 8192), ak4 = MX(64, 2 * K4, 1, 4096, 8192),
                    bk4 = MX(32, 2 * K4, 1, 4096, 8192);
    CHECK(nvfp4_mx_gemm(&ak, &bk, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_mx_gemm(&ak4, &bk4, Y, f32, 32, nat, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED);
    CHECK(nvfp4_mx_gemm(&ak, &bk, Y, f32, 32, NVFP4_MX_ACC_EXACT, NULL, 0, NULL), NVFP4_ERR_UNSUPPORTED);
}

static void misc_cases(void) {
    for (int s = -3; s < 16; ++s)
        if (!nvfp4_status_string((nvfp4_status)s)) ++failures;
    if (nvfp4_version() <= 0) ++failures;
}

int main(void) {
    quantize_cases();
    dequantize_cases();
    requantize_cases();
    gemm_cases();
    mx_cases();
    misc_cases();
    if (failures) {
        fprintf(stderr, "%d mismatches\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
