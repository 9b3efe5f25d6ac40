/*
 * NVFP4 reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of what the NVFP4 quantizer, dequantizer
 * and block-scaled GEMM compute.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The HIP product
 * path never includes, links or calls it, and this code includes nothing from
 * the product path.
 *
 * Sources (web pages; cited by title and section):
 *   [P2] asector.ru, "Nvidia добивается успеха с 4-битным форматом NVFP4",
 *        section "NVFP4 и Blackwell: интеграция архитектуры и формата"
 *        (E2M1 elements in [-6, 6]; a local scale per 16-element block plus a
 *        global scale per tensor; round-to-nearest-even and stochastic
 *        rounding) and section "Эксперименты и сравнение с FP8" (2D weight
 *        scaling, random Hadamard transforms).
 *   [P3] iitak.ru, "Thinking Machines ускорила обучение Inkling 2 Small
 *        4-битными числами", sections "Детали" (the 16-value set, 5 is not
 *        representable; 16-number blocks with a shared multiplier, a block
 *        whose largest magnitude is -54 becomes -6 with multiplier 9),
 *        "Как это работает" (row blocks become column blocks on the
 *        transpose; one multiplier per 16x16 square is transpose-invariant;
 *        random re-rounding of 2.25 to 2 three times in four and to 3 once)
 *        and "В цифрах" (3.6x fewer bits than BF16).
 *
 * What the pages leave open is fixed here (each choice is one plain reading):
 *   - block scale byte: FP8 E4M3 "FN" (bias 7, no infinities, 0x7F unused,
 *     largest finite 448), rounded to nearest-even and clamped at 448;
 *   - tensor scale s_t = A_t / (6 * 448), A_t = largest magnitude of the
 *     tensor being quantized; s_t = 1 when that quotient is 0;
 *   - block multiplier u = A_b / (6 s_t), S = e4m3(u) * s_t, R = 1/S, element
 *     y = |t| * R, all in IEEE binary32 with one rounding per operation;
 *   - stochastic rounding draws a 16-bit integer r per element from
 *     Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *     easy as 1, 2, 3", SC'11) and rounds up iff r < f * 2^16, f being the
 *     position of y between its two neighbouring grid values;
 *   - the Hadamard transform is the 16-point Sylvester matrix scaled by 1/4,
 *     applied after a per-tensor vector of 16 seeded random signs.
 *
 * The MX formats (MXFP8 / MXFP4, and the 8.25-bit transit format) that the
 * pages name without defining follow the OCP Microscaling definition; see the
 * MX section of nvfp4_oracle.c.
 *
 * Parity status of each function is recorded next to it.
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* enum values mirror the public ABI's numbering so that test code can pass
 * the same integers to both sides; the values are restated, not shared. */
enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_ROW_1D = 0, ORC_COL_1D = 1, ORC_ROW_COL_1D = 2, ORC_BLK_2D = 3 };
enum { ORC_RNE = 0, ORC_SR = 1 };
enum { ORC_SCALE_1D = 0, ORC_SCALE_2D = 1 };
/* Philox counter word 2 separates the random streams of the layouts. */
enum { ORC_STREAM_ROW = 0, ORC_STREAM_COL = 1, ORC_STREAM_2D = 2, ORC_STREAM_RHT = 3 };

/* ---- random numbers ---------------------------------------------------- */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t orc_draw16(uint64_t seed, uint32_t stream, uint64_t index);

/* ---- number formats ---------------------------------------------------- */
float orc_e2m1_value(uint32_t code);          /* code 0..15 -> value */
double orc_e4m3_value(uint32_t byte);         /* byte 0..0x7E -> value */
uint32_t orc_e4m3_encode(float u);            /* u >= 0 -> byte */
uint32_t orc_e2m1_rne(float y);               /* y >= 0 -> magnitude code 0..7 */
uint32_t orc_e2m1_sr(float y, uint32_t r16);  /* y >= 0 -> magnitude code 0..7 */
float orc_tensor_scale(float amax);

/* ---- Hadamard transform ------------------------------------------------ */
uint32_t orc_rht_sign_mask(uint64_t seed);
void orc_rht16(const float in[16], uint32_t sign_mask, float out[16]);

/* ---- quantize / dequantize --------------------------------------------- */
/* x: rows x cols, row stride ld elements, dtype ORC_F32 or ORC_BF16 (bits).
 * ROW_1D / BLK_2D outputs: codes rows x cols/2, scales rows x cols/16 (1D)
 * or rows/16 x cols/16 (2D).  COL_1D outputs describe the transpose:
 * codes cols x rows/2, scales cols x rows/16.  ROW_COL_1D writes the row
 * output to (codes, scales, ts) and the column output to (codes2, ...); with
 * the Hadamard transform the row output quantizes x transformed along rows
 * and the column output x transformed along columns, each with its own A_t,
 * and amax_in (when given) points at those two values, the row output's
 * first.
 * index_base is added to every element's linear output index before its
 * random draw, so that a band of a larger tensor can be recomputed alone
 * (0 for a whole tensor).
 * Returns 0 on success, nonzero for an unsupported request. */
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                 int layout, int round, uint64_t sr_seed, int hadamard,
                 uint64_t hadamard_seed, const float* amax_in, uint64_t index_base,
                 uint8_t* codes, uint8_t* scales, float* ts,
                 uint8_t* codes2, uint8_t* scales2, float* ts2);

/* A_t: the largest magnitude of the tensor that `layout` quantizes (after
 * the Hadamard transform along the block dimension when requested). */
float orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int layout,
               int hadamard, uint64_t hadamard_seed);

/* out: rows x cols (stored orientation), dtype ORC_F32 or ORC_BF16 (bits). */
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, float ts,
                    int64_t rows, int64_t cols, int scale_mode, void* out, int out_dtype);

/* Exact dequantize into float64 (v * e4m3(sb) * s_t has <= 30 significant
 * bits, so no rounding happens). */
void orc_dequantize_f64(const uint8_t* codes, const uint8_t* scales, double ts,
                        int64_t rows, int64_t cols, int scale_mode, double* out);

/* C[m,n] = sum_k A[m,k] B[n,k] over exactly dequantized operands, float64,
 * natural k order; W[m,n] = sum_k |A[m,k] B[n,k]|.  If n_entries >= 0 only
 * the listed (m,n) pairs are computed into C[i], W[i]. */
void orc_gemm(const uint8_t* a_codes, const uint8_t* a_scales, double a_ts, int a_mode,
              const uint8_t* b_codes, const uint8_t* b_scales, double b_ts, int b_mode,
              int64_t M, int64_t N, int64_t K,
              const int64_t* entries_m, const int64_t* entries_n, int64_t n_entries,
              double* C, double* W);

/* SwiGLU on float64: h = g * sigmoid(g) * u. */
double orc_swiglu(double g, double u);

/* ---- MX formats (OCP Microscaling; the reading for MXFP8 / MXFP4 and the
 * 8.25-bit transit format): 32-element blocks, E8M0 scale 2^s per block,
 * E4M3 or E2M1 elements; see nvfp4_oracle.c. ------------------------------ */
enum { ORC_MX_FP8 = 0, ORC_MX_FP4 = 1 };
enum { ORC_STREAM_MX_ROW = 4, ORC_STREAM_MX_COL = 5 };
int orc_mx_scale_exp(float amax, int elem);
uint32_t orc_e4m3_sr(float y, uint32_t r16);       /* y >= 0 -> E4M3 byte 0..0x7E */
double orc_mx_elem_value(uint32_t code, int elem);
/* ROW_1D: codes rows x cols (FP8, one byte each) or rows x cols/2 (FP4),
 * scales rows x cols/32; COL_1D describes the transpose.  Returns 0 on
 * success. */
int orc_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int layout,
                    int elem, int round, uint64_t seed, uint64_t index_base, uint8_t* codes,
                    uint8_t* scales);
void orc_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int elem, int64_t rows,
                       int64_t cols, void* out, int out_dtype);
void orc_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int a_elem, const uint8_t* b_codes,
                 const uint8_t* b_scales, int b_elem, int64_t M, int64_t N, int64_t K,
                 const int64_t* entries_m, const int64_t* entries_n, int64_t n_entries, double* C,
                 double* W);

#ifdef __cplusplus
}
#endif
#endif
