/*
 * NVFP4 reference oracle -- TEST INFRASTRUCTURE ONLY (see nvfp4_oracle.h).
 *
 * Plain scalar C, compiled with -O2 -ffp-contract=off and without fast-math:
 * every float operation below is one IEEE binary32 (or binary64 where stated)
 * operation with round-to-nearest-even, in the order written.
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ========================================================================
 * Philox4x32-10.  Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11, section 3 (the Philox S-box and key schedule).
 * Each round multiplies counter words 0 and 2 by the two round multipliers,
 * XORs the high halves with the other two counter words and the round key,
 * and permutes; the key advances by the two Weyl constants between rounds.
 * Parity pin: the Philox4x32-10 engine of the rocRAND library.
 * ====================================================================== */
#define PHILOX_MUL0 0xD2511F53u
#define PHILOX_MUL1 0xCD9E8D57u
#define PHILOX_WEYL0 0x9E3779B9u
#define PHILOX_WEYL1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_WEYL0;
            k1 += PHILOX_WEYL1;
        }
        uint64_t p0 = (uint64_t)PHILOX_MUL0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)PHILOX_MUL1 * (uint64_t)c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Draw for the element with linear index `index` of stream `stream`:
 * counter (index / 8 low, index / 8 high, stream, 0), key (seed low, seed
 * high); element index%8 = j takes 16 bits of word j/2, the low half for
 * even j.  Parity pin: rocRAND engine plus the index mapping test. */
uint32_t orc_draw16(uint64_t seed, uint32_t stream, uint64_t index) {
    uint64_t q = index >> 3;
    uint32_t j = (uint32_t)(index & 7u);
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), stream, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return (w[j >> 1] >> (16u * (j & 1u))) & 0xFFFFu;
}

/* ========================================================================
 * Number formats.
 * ====================================================================== */

/* E2M1: 1 sign, 2 exponent, 1 mantissa bit; magnitudes 0, .5, 1, 1.5, 2, 3,
 * 4, 6 [P2 "NVFP4 и Blackwell"; P3 "Детали"].  Exponent bias 1; exponent
 * field 0 is subnormal with step 0.5.  Parity pin: the value set printed on
 * both pages. */
float orc_e2m1_value(uint32_t code) {
    uint32_t e = (code >> 1) & 3u, m = code & 1u;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

/* E4M3 "FN": bias 7, exponent field 0 subnormal (m * 2^-9), 0x7F unused.
 * The pages only say "local scale"; the FP8 E4M3 encoding is the reading. */
double orc_e4m3_value(uint32_t byte) {
    uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp(1.0 + (double)m / 8.0, (int)e - 7);
}

/* Round u >= 0 to the nearest E4M3 value, ties to the even code, and clamp
 * at the largest finite value 448 (0x7E).  All arithmetic is exact in
 * binary64; nearbyint uses the default ties-to-even mode.  Parity pin:
 * brute-force nearest search over the 127 finite codes. */
uint32_t orc_e4m3_encode(float uf) {
    double u = (double)uf;
    if (!(u > 0.0)) return 0u;
    if (u >= 448.0) return 0x7Eu;
    int e2;
    frexp(u, &e2);           /* u = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;          /* u in [2^e, 2^(e+1)) */
    if (e < -6) {            /* subnormal range: multiples of 2^-9 */
        double q = nearbyint(ldexp(u, 9));
        return (uint32_t)q;  /* q == 8 is the first normal code, 0x08 */
    }
    double m = nearbyint((ldexp(u, -e) - 1.0) * 8.0);
    if (m == 8.0) { m = 0.0; e += 1; }
    return ((uint32_t)(e + 7) << 3) | (uint32_t)m;
}

static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* Round-to-nearest-even onto the E2M1 magnitudes [P2 "NVFP4 и Blackwell"]:
 * the nearest of the eight values; on a tie the even code wins; y >= 6
 * saturates to 6.  Written as the plain nearest search.  Parity pin:
 * RNE(5) = 4 and an exact brute-force over a dense grid. */
uint32_t orc_e2m1_rne(float y) {
    if (y >= 6.0f) return 7u;
    uint32_t best = 0;
    double bestd = fabs((double)y - (double)E2M1_MAG[0]);
    for (uint32_t i = 1; i < 8; ++i) {
        double d = fabs((double)y - (double)E2M1_MAG[i]);
        if (d < bestd || (d == bestd && (i & 1u) == 0u)) {
            best = i;
            bestd = d;
        }
    }
    return best;
}

/* Stochastic rounding [P2 "NVFP4 и Blackwell"; P3 "Как это работает"]: with
 * lo <= y < hi the neighbouring grid values and f = (y - lo) / (hi - lo),
 * round up iff r16 < f * 2^16, so that P(up) = f up to 2^-16 and the mean of
 * the result is y.  Evaluated exactly in binary64.  Parity pin: the 2.25 ->
 * 2 or 3 example (probability 1/4 exactly) and exhaustive counts over r16. */
uint32_t orc_e2m1_sr(float y, uint32_t r16) {
    if (y >= 6.0f) return 7u;
    uint32_t lo = 0;
    for (uint32_t i = 1; i < 8; ++i)
        if ((double)E2M1_MAG[i] <= (double)y) lo = i;
    double f = ((double)y - (double)E2M1_MAG[lo]) /
               ((double)E2M1_MAG[lo + 1] - (double)E2M1_MAG[lo]);
    return ((double)r16 < f * 65536.0) ? lo + 1 : lo;
}

/* Global (per-tensor) scale: s_t = A_t / (6 * 448) in binary32, so that the
 * tensor's largest block gets the largest E4M3 multiplier [P2: local scale
 * per 16-element block plus a global per-tensor scale].  s_t = 1 when the
 * quotient is 0 (an all-zero tensor, or underflow). */
float orc_tensor_scale(float amax) {
    float st = amax / 2688.0f;
    return (st > 0.0f) ? st : 1.0f;
}

/* ========================================================================
 * 16-point random Hadamard transform [P2 "Эксперименты и сравнение с FP8":
 * random Hadamard transforms for stability].  t = (1/4) H16 D x with H16 the
 * Sylvester matrix H[i][j] = (-1)^popcount(i & j) and D = diag(d), d_i = -1
 * iff bit i of the sign mask is set.  Evaluated as four butterfly stages
 * (h = 1, 2, 4, 8; pair (i, i+h) -> (sum, difference)) then a scale by 1/4,
 * each step one binary32 operation.  Parity pin: d = +1 reproduces the
 * textbook Walsh-Hadamard matrix; inverse, Parseval and dot products.
 * ====================================================================== */
uint32_t orc_rht_sign_mask(uint64_t seed) {
    uint32_t ctr[4] = {0u, 0u, ORC_STREAM_RHT, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return w[0] & 0xFFFFu;
}

void orc_rht16(const float in[16], uint32_t sign_mask, float out[16]) {
    float z[16];
    for (int i = 0; i < 16; ++i) z[i] = ((sign_mask >> i) & 1u) ? -in[i] : in[i];
    for (int h = 1; h < 16; h <<= 1) {
        for (int i = 0; i < 16; ++i) {
            if (i & h) continue;
            float a = z[i], b = z[i + h];
            z[i] = a + b;
            z[i + h] = a - b;
        }
    }
    for (int i = 0; i < 16; ++i) out[i] = 0.25f * z[i];
}

/* ========================================================================
 * Quantization.
 * ====================================================================== */

static float load_elem(const void* x, int dtype, int64_t idx) {
    if (dtype == ORC_BF16) {
        uint32_t b = (uint32_t)((const uint16_t*)x)[idx] << 16;
        float f;
        memcpy(&f, &b, 4);
        return f;
    }
    return ((const float*)x)[idx];
}

/* Per-block parameters [P3 "Детали": the block's largest magnitude maps to
 * 6, so the multiplier is A_b / 6]: u = A_b / (6 s_t) rounded to E4M3, the
 * block multiplier S = e4m3(u) * s_t and its reciprocal R. */
typedef struct { uint32_t byte; float S, R; } blockscale;

static blockscale block_scale(float amax_b, float st) {
    blockscale b;
    float denom = 6.0f * st;
    float u = amax_b / denom;
    b.byte = orc_e4m3_encode(u);
    b.S = (float)orc_e4m3_value(b.byte) * st;
    b.R = (b.S > 0.0f) ? 1.0f / b.S : 0.0f;
    return b;
}

/* Encode one element t with block parameters b; `index` is the element's
 * linear index in the output tensor (the counter of its random draw). */
static uint32_t encode_elem(float t, blockscale b, int round, uint64_t seed,
                            uint32_t stream, uint64_t index) {
    uint32_t sign = signbit(t) ? 8u : 0u;
    if (b.S == 0.0f || t == 0.0f) return sign;
    float y = fabsf(t) * b.R;
    uint32_t mag = (round == ORC_SR) ? orc_e2m1_sr(y, orc_draw16(seed, stream, index))
                                     : orc_e2m1_rne(y);
    return sign | mag;
}

static void put_code(uint8_t* codes, int64_t cols, int64_t r, int64_t c, uint32_t code) {
    uint8_t* p = &codes[r * (cols / 2) + c / 2];
    if (c & 1) *p = (uint8_t)((*p & 0x0Fu) | (code << 4));
    else *p = (uint8_t)((*p & 0xF0u) | code);
}

/* 1D quantization of the oriented tensor t [R x C] (fp32, dense): blocks of
 * 16 consecutive elements along each row [P3 "Детали"]. */
static void quantize_rows(const float* t, int64_t R, int64_t C, float amax_t, int round,
                          uint64_t seed, uint32_t stream, uint64_t index_base, uint8_t* codes,
                          uint8_t* scales, float* ts) {
    float st = orc_tensor_scale(amax_t);
    *ts = st;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t c0 = 0; c0 < C; c0 += 16) {
            float ab = 0.0f;
            for (int64_t c = c0; c < c0 + 16; ++c) ab = fmaxf(ab, fabsf(t[r * C + c]));
            blockscale b = block_scale(ab, st);
            scales[r * (C / 16) + c0 / 16] = (uint8_t)b.byte;
            for (int64_t c = c0; c < c0 + 16; ++c)
                put_code(codes, C, r, c,
                         encode_elem(t[r * C + c], b, round, seed, stream,
                                     index_base + (uint64_t)(r * C + c)));
        }
    }
}

/* 2D quantization: one scale per 16 x 16 square [P2 "Эксперименты и сравнение
 * с FP8": 2D weight scaling; P3 "Как это работает": one multiplier per 16x16
 * square, unchanged by the transpose]. */
static void quantize_2d(const float* t, int64_t R, int64_t C, float amax_t, int round,
                        uint64_t seed, uint64_t index_base, uint8_t* codes, uint8_t* scales,
                        float* ts) {
    float st = orc_tensor_scale(amax_t);
    *ts = st;
    for (int64_t r0 = 0; r0 < R; r0 += 16) {
        for (int64_t c0 = 0; c0 < C; c0 += 16) {
            float ab = 0.0f;
            for (int64_t r = r0; r < r0 + 16; ++r)
                for (int64_t c = c0; c < c0 + 16; ++c) ab = fmaxf(ab, fabsf(t[r * C + c]));
            blockscale b = block_scale(ab, st);
            scales[(r0 / 16) * (C / 16) + c0 / 16] = (uint8_t)b.byte;
            for (int64_t r = r0; r < r0 + 16; ++r)
                for (int64_t c = c0; c < c0 + 16; ++c)
                    put_code(codes, C, r, c,
                             encode_elem(t[r * C + c], b, round, seed, ORC_STREAM_2D,
                                         index_base + (uint64_t)(r * C + c)));
        }
    }
}

static float amax_of(const float* t, int64_t n) {
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) a = fmaxf(a, fabsf(t[i]));
    return a;
}

/* Build the oriented fp32 tensor: x itself (ROW) or its transpose (COL, the
 * column-wise re-quantization [P3 "Как это работает"]), then the optional
 * Hadamard transform on every aligned 16-chunk of each oriented row. */
static float* oriented(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                       int transpose, int hadamard, uint64_t hseed) {
    int64_t R = transpose ? cols : rows, C = transpose ? rows : cols;
    float* t = (float*)malloc((size_t)(R * C) * sizeof(float));
    if (!t) return NULL;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = load_elem(x, dtype, r * ld + c);
            if (transpose) t[c * C + r] = v;
            else t[r * C + c] = v;
        }
    if (hadamard) {
        uint32_t mask = orc_rht_sign_mask(hseed);
        for (int64_t r = 0; r < R; ++r)
            for (int64_t c0 = 0; c0 < C; c0 += 16) orc_rht16(&t[r * C + c0], mask, &t[r * C + c0]);
    }
    return t;
}

int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 int layout, int round, uint64_t sr_seed, int hadamard,
                 uint64_t hadamard_seed, const float* amax_in, uint64_t index_base,
                 uint8_t* codes, uint8_t* scales, float* ts,
                 uint8_t* codes2, uint8_t* scales2, float* ts2) {
    if (rows < 0 || cols < 0 || ld < cols) return 1;
    if (layout == ORC_BLK_2D && hadamard) return 2;
    if ((layout == ORC_ROW_1D || layout == ORC_ROW_COL_1D || layout == ORC_BLK_2D) && cols % 16) return 3;
    if ((layout == ORC_COL_1D || layout == ORC_ROW_COL_1D || layout == ORC_BLK_2D) && rows % 16) return 3;

    if (layout == ORC_ROW_1D || layout == ORC_COL_1D) {
        int tr = (layout == ORC_COL_1D);
        float* t = oriented(x, dtype, rows, cols, ld, tr, hadamard, hadamard_seed);
        if (!t && rows > 0 && cols > 0) return 4;
        int64_t R = tr ? cols : rows, C = tr ? rows : cols;
        float a = amax_in ? *amax_in : amax_of(t, R * C);
        quantize_rows(t, R, C, a, round, sr_seed, tr ? ORC_STREAM_COL : ORC_STREAM_ROW,
                      index_base, codes, scales, ts);
        free(t);
        return 0;
    }
    if (layout == ORC_ROW_COL_1D) {
        /* Both orientations of one tensor.  Without the transform they share
         * one A_t.  With it, the row output is ROW_1D of the tensor transformed
         * along rows and the column output COL_1D of the tensor transformed
         * along columns: two different tensors, each with its own A_t
         * (amax_in then holds two values, the row output's first). */
        float* t = oriented(x, dtype, rows, cols, ld, 0, hadamard, hadamard_seed);
        float* tt = oriented(x, dtype, rows, cols, ld, 1, hadamard, hadamard_seed);
        if ((!t || !tt) && rows > 0 && cols > 0) { free(t); free(tt); return 4; }
        float a = amax_in ? amax_in[0] : amax_of(t, rows * cols);
        float a2 = !hadamard ? a : amax_in ? amax_in[1] : amax_of(tt, rows * cols);
        quantize_rows(t, rows, cols, a, round, sr_seed, ORC_STREAM_ROW, index_base, codes, scales,
                      ts);
        quantize_rows(tt, cols, rows, a2, round, sr_seed, ORC_STREAM_COL, index_base, codes2,
                      scales2, ts2);
        free(t);
        free(tt);
        return 0;
    }
    if (layout == ORC_BLK_2D) {
        float* t = oriented(x, dtype, rows, cols, ld, 0, 0, 0);
        if (!t && rows > 0 && cols > 0) return 4;
        float a = amax_in ? *amax_in : amax_of(t, rows * cols);
        quantize_2d(t, rows, cols, a, round, sr_seed, index_base, codes, scales, ts);
        free(t);
        return 0;
    }
    return 5;
}

float orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int layout,
               int hadamard, uint64_t hadamard_seed) {
    int tr = (layout == ORC_COL_1D);
    float* t = oriented(x, dtype, rows, cols, ld, tr, hadamard, hadamard_seed);
    if (!t) return 0.0f;
    float a = amax_of(t, rows * cols);
    free(t);
    return a;
}

/* ========================================================================
 * Dequantization: back to a wider format [P3 "Как это работает": the values
 * are converted to a more precise format before re-rounding].
 * x = v * e4m3(sb) * s_t; v * e4m3(sb) has at most 6 significant bits and is
 * exact in binary32, so one rounding happens (at * s_t); BF16 output is the
 * nearest-even BF16 of that binary32 value.
 * ====================================================================== */
static uint8_t scale_byte(const uint8_t* scales, int64_t r, int64_t c, int64_t cols, int mode) {
    if (mode == ORC_SCALE_2D) return scales[(r / 16) * (cols / 16) + c / 16];
    return scales[r * (cols / 16) + c / 16];
}

static uint32_t get_code(const uint8_t* codes, int64_t cols, int64_t r, int64_t c) {
    uint8_t b = codes[r * (cols / 2) + c / 2];
    return (c & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 0x0Fu);
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    /* finite inputs only: add half an ulp of bf16 plus the tie-to-even bit */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void orc_dequantize(const uint8_t* codes, const uint8_t* scales, float ts,
                    int64_t rows, int64_t cols, int scale_mode, void* out, int out_dtype) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float v = orc_e2m1_value(get_code(codes, cols, r, c));
            float sb = (float)orc_e4m3_value(scale_byte(scales, r, c, cols, scale_mode));
            float p = v * sb;   /* exact */
            float x = p * ts;
            if (out_dtype == ORC_BF16) ((uint16_t*)out)[r * cols + c] = f32_to_bf16_rne(x);
            else ((float*)out)[r * cols + c] = x;
        }
}

void orc_dequantize_f64(const uint8_t* codes, const uint8_t* scales, double ts,
                        int64_t rows, int64_t cols, int scale_mode, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double v = (double)orc_e2m1_value(get_code(codes, cols, r, c));
            double sb = orc_e4m3_value(scale_byte(scales, r, c, cols, scale_mode));
            out[r * cols + c] = v * sb * ts;
        }
}

/* ========================================================================
 * Block-scaled GEMM reference [P2 "NVFP4 и Blackwell": scaled compute with
 * high-precision accumulation]: the plain definition on exactly dequantized
 * operands, C = A B^T, accumulated in binary64 in natural k order.
 * Parity pin: brute force on tiny shapes; the exact all-unit-scale case.
 * ====================================================================== */
static double deq(const uint8_t* codes, const uint8_t* scales, double ts, int mode,
                  int64_t cols, int64_t r, int64_t c) {
    double v = (double)orc_e2m1_value(get_code(codes, cols, r, c));
    double sb = orc_e4m3_value(scale_byte(scales, r, c, cols, mode));
    return v * sb * ts;
}

static void gemm_entry(const uint8_t* ac, const uint8_t* as, double ats, int am,
                       const uint8_t* bc, const uint8_t* bs, double bts, int bm,
                       int64_t K, int64_t m, int64_t n, double* c, double* w) {
    double acc = 0.0, wacc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = deq(ac, as, ats, am, K, m, k) * deq(bc, bs, bts, bm, K, n, k);
        acc += p;
        wacc += fabs(p);
    }
    *c = acc;
    *w = wacc;
}

void orc_gemm(const uint8_t* a_codes, const uint8_t* a_scales, double a_ts, int a_mode,
              const uint8_t* b_codes, const uint8_t* b_scales, double b_ts, int b_mode,
              int64_t M, int64_t N, int64_t K,
              const int64_t* entries_m, const int64_t* entries_n, int64_t n_entries,
              double* C, double* W) {
    if (n_entries >= 0) {
        for (int64_t i = 0; i < n_entries; ++i)
            gemm_entry(a_codes, a_scales, a_ts, a_mode, b_codes, b_scales, b_ts, b_mode, K,
                       entries_m[i], entries_n[i], &C[i], &W[i]);
        return;
    }
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_entry(a_codes, a_scales, a_ts, a_mode, b_codes, b_scales, b_ts, b_mode, K,
                       m, n, &C[m * N + n], &W[m * N + n]);
}

/* SwiGLU: gate * sigmoid(gate) * up, in binary64. */
double orc_swiglu(double g, double u) {
    return g / (1.0 + exp(-g)) * u;
}

/* ========================================================================
 * MX formats (OCP Microscaling).
 *
 * The pages name MXFP8 (the backward pass at Thinking Machines runs in it:
 * P3 "Как это работает"; Blackwell tensor cores support MXFP8/MXFP6/MXFP4:
 * P2 "NVFP4 и Blackwell"), MXFP4 (the Open Compute Project's 4-bit format
 * NVFP4 is compared with: P1; P2 "Перспективы и дальнейшие направления
 * исследований") and an 8.25-bit transit format for expert outputs (P3
 * "Но"), but define none of them.  The reading here is the OCP Microscaling definition: blocks of 32
 * consecutive elements along the block dimension share one E8M0 scale
 * X = 2^s, s = floor(log2(max |V|)) - emax (emax = 8 for E4M3 elements,
 * 2 for E2M1), clamped to [-127, 127] (s = -127 for an all-zero block);
 * element P = round(V / X) onto the element format with saturation at its
 * largest finite value (448 or 6).  As for NVFP4 every step is binary32 with
 * one rounding: y = fl(|V| * 2^-s) (a multiply by an exact power of two),
 * then y is rounded to nearest-even or stochastically with a 16-bit Philox
 * draw (round up iff r16 < f * 2^16, f the position of y between its grid
 * neighbours), the sign copied.  The 8-bit element and 8-bit scale per 32
 * give 8 + 8/32 = 8.25 bits per number (P3 "Но").
 * ====================================================================== */

/* floor(log2(a)) - emax clamped to [-127, 127]; -127 when a == 0. */
int orc_mx_scale_exp(float amax, int elem) {
    if (!(amax > 0.0f)) return -127;
    int e;
    frexpf(amax, &e);                      /* amax = f * 2^e, f in [0.5, 1) */
    int s = (e - 1) - (elem == ORC_MX_FP8 ? 8 : 2);
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    return s;
}

/* E4M3 stochastic rounding of y >= 0 (y >= 448 saturates to 0x7E): lo = the
 * largest finite E4M3 value <= y (found by a plain search over the codes),
 * hi the next one, round up iff r16 < f * 2^16.  Exact in binary64. */
uint32_t orc_e4m3_sr(float yf, uint32_t r16) {
    double y = (double)yf;
    if (y >= 448.0) return 0x7Eu;
    uint32_t lo = 0;
    for (uint32_t b = 1; b <= 0x7Eu; ++b)
        if (orc_e4m3_value(b) <= y) lo = b;
    double vlo = orc_e4m3_value(lo), vhi = orc_e4m3_value(lo + 1);
    double f = (y - vlo) / (vhi - vlo);
    return ((double)r16 < f * 65536.0) ? lo + 1 : lo;
}

/* Value of an MX element code: E4M3 byte (sign in bit 7) or E2M1 nibble. */
double orc_mx_elem_value(uint32_t code, int elem) {
    if (elem == ORC_MX_FP8) {
        double v = orc_e4m3_value(code & 0x7Fu);
        return (code & 0x80u) ? -v : v;
    }
    return (double)orc_e2m1_value(code & 15u);
}

static uint32_t mx_encode(float v, float p2, int elem, int round, uint64_t seed, uint32_t stream,
                          uint64_t index) {
    float y = fabsf(v) * p2;
    uint32_t r16 = round == ORC_SR ? orc_draw16(seed, stream, index) : 0u;
    if (elem == ORC_MX_FP8) {
        uint32_t sign = signbit(v) ? 0x80u : 0u;
        uint32_t mag = round == ORC_SR ? orc_e4m3_sr(y, r16) : orc_e4m3_encode(y);
        return sign | mag;
    }
    uint32_t sign = signbit(v) ? 8u : 0u;
    return sign | (round == ORC_SR ? orc_e2m1_sr(y, r16) : orc_e2m1_rne(y));
}

int orc_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int layout,
                    int elem, int round, uint64_t seed, uint64_t index_base, uint8_t* codes,
                    uint8_t* scales) {
    if (layout != ORC_ROW_1D && layout != ORC_COL_1D) return 1;
    if (elem != ORC_MX_FP8 && elem != ORC_MX_FP4) return 2;
    const int transpose = layout == ORC_COL_1D;
    const int64_t R = transpose ? cols : rows, C = transpose ? rows : cols;
    if (C % 32) return 3;
    float* t = oriented(x, dtype, rows, cols, ld, transpose, 0, 0);
    if (!t) return 4;
    const uint32_t stream = transpose ? ORC_STREAM_MX_COL : ORC_STREAM_MX_ROW;
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t c0 = 0; c0 < C; c0 += 32) {
            float ab = 0.0f;
            for (int64_t c = c0; c < c0 + 32; ++c) ab = fmaxf(ab, fabsf(t[r * C + c]));
            int s = orc_mx_scale_exp(ab, elem);
            scales[r * (C / 32) + c0 / 32] = (uint8_t)(s + 127);
            float p2 = ldexpf(1.0f, -s);   /* exact: 2^-127 .. 2^127 */
            for (int64_t c = c0; c < c0 + 32; ++c) {
                uint32_t code = mx_encode(t[r * C + c], p2, elem, round, seed, stream,
                                          index_base + (uint64_t)(r * C + c));
                if (elem == ORC_MX_FP8) codes[r * C + c] = (uint8_t)code;
                else put_code(codes, C, r, c, code);
            }
        }
    }
    free(t);
    return 0;
}

static double mx_deq(const uint8_t* codes, const uint8_t* scales, int elem, int64_t cols, int64_t r,
                     int64_t c) {
    uint32_t code = elem == ORC_MX_FP8 ? codes[r * cols + c] : get_code(codes, cols, r, c);
    int s = (int)scales[r * (cols / 32) + c / 32] - 127;
    return ldexp(orc_mx_elem_value(code, elem), s);   /* exact */
}

/* out: rows x cols, ORC_F32 (the exact value, which binary32 holds), ORC_BF16
 * (nearest-even of that value) or float64 when out_dtype == 2. */
void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int elem, int64_t rows,
                       int64_t cols, void* out, int out_dtype) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double v = mx_deq(codes, scales, elem, cols, r, c);
            if (out_dtype == 2) ((double*)out)[r * cols + c] = v;
            else if (out_dtype == ORC_BF16) ((uint16_t*)out)[r * cols + c] = f32_to_bf16_rne((float)v);
            else ((float*)out)[r * cols + c] = (float)v;
        }
}

/* C[m,n] = sum_k A[m,k] B[n,k] over exactly dequantized MX operands (the
 * block-scaled MMA the pages describe for Blackwell, P2 "NVFP4 и
 * Blackwell"), float64, natural k order; W = sum |a b|; entries as orc_gemm. */
void orc_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int a_elem, const uint8_t* b_codes,
                 const uint8_t* b_scales, int b_elem, int64_t M, int64_t N, int64_t K,
                 const int64_t* entries_m, const int64_t* entries_n, int64_t n_entries, double* C,
                 double* W) {
    int64_t count = n_entries >= 0 ? n_entries : M * N;
    for (int64_t i = 0; i < count; ++i) {
        int64_t m = n_entries >= 0 ? entries_m[i] : i / N;
        int64_t n = n_entries >= 0 ? entries_n[i] : i % N;
        double acc = 0.0, wacc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = mx_deq(a_codes, a_scales, a_elem, K, m, k) * mx_deq(b_codes, b_scales, b_elem, K, n, k);
            acc += p;
            wacc += fabs(p);
        }
        C[i] = acc;
        W[i] = wacc;
    }
}
