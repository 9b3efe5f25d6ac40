/*
 * Memory and undefined-behaviour check of the CPU oracle (test infrastructure
 * only): tests/test_oracle_sanitize.py builds this file together with
 * oracle/nvfp4_oracle.c under gcc's AddressSanitizer and UndefinedBehavior-
 * Sanitizer (host code only; nothing here runs on a GPU) and runs it.
 *
 * Every entry point of oracle/nvfp4_oracle.h is called on small inputs whose
 * buffers are allocated at exactly the sizes the header documents, so a read
 * or write one element past an input or output is reported; the shapes cover
 * ragged sizes, row strides larger than the width, both input types, both
 * roundings, the Hadamard transform and every layout, and the values include
 * zeros of both signs, binary32 subnormals and magnitudes near the binary32
 * maximum.  The program prints one line per group of calls and "ok" at the
 * end; any sanitizer report ends it with a nonzero status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../oracle/nvfp4_oracle.h"

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) {
    lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(lcg_state >> 32);
}

/* A value of one of several kinds: ordinary, zero, -0, subnormal, large. */
static float next_value(void) {
    const uint32_t k = next_u32() % 16u;
    const float u = (float)(next_u32() >> 8) / 16777216.0f - 0.5f;  /* [-0.5, 0.5) */
    if (k == 0) return 0.0f;
    if (k == 1) return -0.0f;
    if (k == 2) return u * 1e-40f;          /* subnormal */
    if (k == 3) return (float)(u * 6.0e38);  /* up to 3e38, near the binary32 maximum */
    if (k == 4) return u * 1e-30f;
    return u * 8.0f;
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(3);
    }
    return p;
}

/* rows x cols input with row stride ld, F32 or BF16 bits; exactly rows*ld elements */
static void* make_input(int dtype, int64_t rows, int64_t ld) {
    const size_t n = (size_t)(rows * ld);
    if (dtype == ORC_F32) {
        float* x = xmalloc(n * sizeof(float));
        for (size_t i = 0; i < n; ++i) x[i] = next_value();
        return x;
    }
    uint16_t* x = xmalloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        const float v = next_value();
        uint32_t b;
        memcpy(&b, &v, 4);
        x[i] = (uint16_t)(b >> 16);  /* truncation: any BF16 pattern will do here */
    }
    return x;
}

static void check_rc(int rc, const char* what) {
    if (rc != 0) {
        fprintf(stderr, "unexpected rejection (%d): %s\n", rc, what);
        exit(4);
    }
}

static void quantize_cases(void) {
    static const int64_t shapes[][3] = {{16, 16, 16}, {16, 16, 24}, {32, 48, 48}, {48, 80, 96}, {64, 32, 40}, {0, 16, 16}, {16, 0, 0}};
    const int nshape = (int)(sizeof(shapes) / sizeof(shapes[0]));
    int calls = 0;
    for (int s = 0; s < nshape; ++s) {
        const int64_t rows = shapes[s][0], cols = shapes[s][1], ld = shapes[s][2];
        for (int dtype = 0; dtype < 2; ++dtype) {
            void* x = make_input(dtype, rows, ld);
            for (int layout = ORC_ROW_1D; layout <= ORC_BLK_2D; ++layout) {
                for (int round = ORC_RNE; round <= ORC_SR; ++round) {
                    for (int had = 0; had < 2; ++had) {
                        if (layout == ORC_BLK_2D && had) continue;
                        const int col = layout == ORC_COL_1D;
                        const int64_t R = col ? cols : rows, C = col ? rows : cols;
                        const size_t ncodes = (size_t)(R * (C / 2));
                        const size_t nscales = layout == ORC_BLK_2D ? (size_t)((R / 16) * (C / 16)) : (size_t)(R * (C / 16));
                        uint8_t* codes = xmalloc(ncodes);
                        uint8_t* scales = xmalloc(nscales);
                        float ts = 0.0f, ts2 = 0.0f;
                        uint8_t* codes2 = NULL;
                        uint8_t* scales2 = NULL;
                        if (layout == ORC_ROW_COL_1D) {
                            codes2 = xmalloc((size_t)(cols * (rows / 2)));
                            scales2 = xmalloc((size_t)(cols * (rows / 16)));
                        }
                        check_rc(orc_quantize(x, dtype, rows, cols, ld, layout, round, 1234u + (uint64_t)s, had, 77u,
                                              NULL, 0, codes, scales, &ts, codes2, scales2, &ts2),
                                 "orc_quantize");
                        /* with a caller-supplied A_t (and an index base) as well */
                        float am[2];
                        am[0] = orc_amax(x, dtype, rows, cols, ld, layout == ORC_ROW_COL_1D ? ORC_ROW_1D : layout, had, 77u);
                        am[1] = orc_amax(x, dtype, rows, cols, ld, layout == ORC_ROW_COL_1D ? ORC_COL_1D : layout, had, 77u);
                        check_rc(orc_quantize(x, dtype, rows, cols, ld, layout, round, 99u, had, 77u, am, 4096u, codes,
                                              scales, &ts, codes2, scales2, &ts2),
                                 "orc_quantize amax_in");
                        calls += 2;
                        /* dequantize the stored result into both output types */
                        const int mode = layout == ORC_BLK_2D ? ORC_SCALE_2D : ORC_SCALE_1D;
                        float* yf = xmalloc((size_t)(R * C) * sizeof(float));
                        uint16_t* yb = xmalloc((size_t)(R * C) * sizeof(uint16_t));
                        double* yd = xmalloc((size_t)(R * C) * sizeof(double));
                        orc_dequantize(codes, scales, ts, R, C, mode, yf, ORC_F32);
                        orc_dequantize(codes, scales, ts, R, C, mode, yb, ORC_BF16);
                        orc_dequantize_f64(codes, scales, (double)ts, R, C, mode, yd);
                        calls += 3;
                        free(yf);
                        free(yb);
                        free(yd);
                        free(codes);
                        free(scales);
                        free(codes2);
                        free(scales2);
                    }
                }
            }
            /* unsupported requests are refused without touching the outputs */
            if (orc_quantize(x, dtype, rows, cols, ld, ORC_BLK_2D, ORC_RNE, 0, 1, 0, NULL, 0, NULL, NULL, NULL,
                             NULL, NULL, NULL) == 0) {
                fprintf(stderr, "BLK_2D with the transform was accepted\n");
                exit(4);
            }
            free(x);
        }
    }
    printf("quantize / amax / dequantize: %d calls\n", calls);
}

static void gemm_cases(void) {
    static const int64_t mnk[][3] = {{1, 1, 16}, {16, 32, 48}, {33, 17, 64}, {0, 4, 16}};
    int calls = 0;
    for (int s = 0; s < 4; ++s) {
        const int64_t M = mnk[s][0], N = mnk[s][1], K = mnk[s][2];
        for (int bmode = ORC_SCALE_1D; bmode <= ORC_SCALE_2D; ++bmode) {
            const int64_t Np = bmode == ORC_SCALE_2D ? (N + 15) / 16 * 16 : N;  /* 2D needs rows % 16 */
            float* a = make_input(ORC_F32, M, K);
            float* b = make_input(ORC_F32, Np, K);
            uint8_t* ac = xmalloc((size_t)(M * (K / 2)));
            uint8_t* as = xmalloc((size_t)(M * (K / 16)));
            uint8_t* bc = xmalloc((size_t)(Np * (K / 2)));
            uint8_t* bs = xmalloc(bmode == ORC_SCALE_2D ? (size_t)((Np / 16) * (K / 16)) : (size_t)(Np * (K / 16)));
            float ats = 0.0f, bts = 0.0f;
            check_rc(orc_quantize(a, ORC_F32, M, K, K, ORC_ROW_1D, ORC_RNE, 0, 0, 0, NULL, 0, ac, as, &ats, NULL, NULL,
                                  NULL),
                     "gemm A");
            check_rc(orc_quantize(b, ORC_F32, Np, K, K, bmode == ORC_SCALE_2D ? ORC_BLK_2D : ORC_ROW_1D, ORC_RNE, 0,
                                  0, 0, NULL, 0, bc, bs, &bts, NULL, NULL, NULL),
                     "gemm B");
            double* C = xmalloc((size_t)(M * Np) * sizeof(double));
            double* W = xmalloc((size_t)(M * Np) * sizeof(double));
            orc_gemm(ac, as, ats, ORC_SCALE_1D, bc, bs, bts, bmode, M, Np, K, NULL, NULL, -1, C, W);
            int64_t em[3], en[3];
            const int64_t ne = M > 0 ? 3 : 0;
            for (int64_t i = 0; i < ne; ++i) {
                em[i] = (int64_t)(next_u32() % (uint32_t)M);
                en[i] = (int64_t)(next_u32() % (uint32_t)Np);
            }
            double Ce[3], We[3];
            orc_gemm(ac, as, ats, ORC_SCALE_1D, bc, bs, bts, bmode, M, Np, K, em, en, ne, Ce, We);
            calls += 2;
            double acc = 0.0;
            for (int64_t i = 0; i < M * Np; ++i) acc += W[i];
            if (M * Np > 0) acc += orc_swiglu(C[0], 1.0);
            (void)acc;
            free(a);
            free(b);
            free(ac);
            free(as);
            free(bc);
            free(bs);
            free(C);
            free(W);
        }
    }
    printf("gemm: %d calls\n", calls);
}

static void mx_cases(void) {
    static const int64_t shapes[][3] = {{32, 32, 32}, {64, 96, 104}, {32, 64, 64}, {0, 32, 32}};
    int calls = 0;
    for (int s = 0; s < 4; ++s) {
        const int64_t rows = shapes[s][0], cols = shapes[s][1], ld = shapes[s][2];
        for (int dtype = 0; dtype < 2; ++dtype) {
            void* x = make_input(dtype, rows, ld);
            for (int layout = ORC_ROW_1D; layout <= ORC_COL_1D; ++layout) {
                for (int elem = ORC_MX_FP8; elem <= ORC_MX_FP4; ++elem) {
                    for (int round = ORC_RNE; round <= ORC_SR; ++round) {
                        const int col = layout == ORC_COL_1D;
                        const int64_t R = col ? cols : rows, C = col ? rows : cols;
                        const int64_t cb = elem == ORC_MX_FP8 ? C : C / 2;
                        uint8_t* codes = xmalloc((size_t)(R * cb));
                        uint8_t* scales = xmalloc((size_t)(R * (C / 32)));
                        check_rc(orc_mx_quantize(x, dtype, rows, cols, ld, layout, elem, round, 5u, 0, codes, scales),
                                 "orc_mx_quantize");
                        float* yf = xmalloc((size_t)(R * C) * sizeof(float));
                        uint16_t* yb = xmalloc((size_t)(R * C) * sizeof(uint16_t));
                        orc_mx_dequantize(codes, scales, elem, R, C, yf, ORC_F32);
                        orc_mx_dequantize(codes, scales, elem, R, C, yb, ORC_BF16);
                        double* Cm = xmalloc((size_t)(R * R) * sizeof(double));
                        double* Wm = xmalloc((size_t)(R * R) * sizeof(double));
                        orc_mx_gemm(codes, scales, elem, codes, scales, elem, R, R, C, NULL, NULL, -1, Cm, Wm);
                        calls += 4;
                        free(yf);
                        free(yb);
                        free(Cm);
                        free(Wm);
                        free(codes);
                        free(scales);
                    }
                }
            }
            free(x);
        }
    }
    printf("mx quantize / dequantize / gemm: %d calls\n", calls);
}

static void scalar_cases(void) {
    uint32_t acc = 0;
    for (uint32_t c = 0; c < 16; ++c) acc += (uint32_t)(orc_e2m1_value(c) > 0.0f);
    for (uint32_t b = 0; b < 0x7F; ++b) acc += (uint32_t)(orc_e4m3_value(b) > 1.0);
    for (int i = 0; i < 200000; ++i) {
        const float v = next_value();
        const float a = v < 0.0f ? -v : v;
        acc += orc_e4m3_encode(a) + orc_e2m1_rne(a) + orc_e2m1_sr(a, next_u32() & 0xFFFFu);
        acc += orc_e4m3_sr(a, next_u32() & 0xFFFFu) + (uint32_t)orc_mx_scale_exp(a, (int)(i & 1));
        acc += (uint32_t)(orc_tensor_scale(a) > 1.0f);
    }
    for (uint32_t c = 0; c < 256; ++c) acc += (uint32_t)(orc_mx_elem_value(c, ORC_MX_FP8) > 0.0);
    for (uint32_t c = 0; c < 16; ++c) acc += (uint32_t)(orc_mx_elem_value(c, ORC_MX_FP4) > 0.0);
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
    orc_philox4x32_10(ctr, key, out);
    acc += out[0] + orc_draw16(~0ull, ORC_STREAM_COL, ~0ull);
    float in[16], o16[16];
    for (int i = 0; i < 16; ++i) in[i] = next_value();
    orc_rht16(in, orc_rht_sign_mask(12345u), o16);
    printf("scalar functions: checksum %u\n", acc);
}

int main(void) {
    quantize_cases();
    gemm_cases();
    mx_cases();
    scalar_cases();
    printf("ok\n");
    return 0;
}
