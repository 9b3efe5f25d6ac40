/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 library: block-scaled 4-bit
 * quantization and the block-scaled GEMMs that consume it.
 *
 * The format (sources are web pages, cited by title and section):
 *   - elements are E2M1 codes: 1 sign, 2 exponent and 1 mantissa bit, values
 *     +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} ("Nvidia добивается успеха с 4-битным
 *     форматом NVFP4", asector.ru, section "NVFP4 и Blackwell: интеграция
 *     архитектуры и формата"; "Thinking Machines ускорила обучение Inkling 2
 *     Small 4-битными числами", iitak.ru, section "Детали");
 *   - two scale levels: one multiplier per block of 16 elements and one per
 *     tensor (asector.ru page, same section); the block multiplier maps the
 *     block's largest magnitude to 6, e.g. -54 becomes -6 with multiplier 9
 *     (iitak.ru page, "Детали");
 *   - blocks run along rows, along columns (the re-quantization of the
 *     transpose that the backward pass needs), or over 16x16 squares whose
 *     multiplier is unchanged by a transpose (iitak.ru page, "Как это
 *     работает"; asector.ru page, "Эксперименты и сравнение с FP8");
 *   - rounding is to nearest-even or stochastic (asector.ru page, "NVFP4 и
 *     Blackwell"; the 2.25 -> 2 or 3 example on the iitak.ru page, "Как это
 *     работает");
 *   - an optional random Hadamard transform precedes quantization
 *     (asector.ru page, "Эксперименты и сравнение с FP8").
 *
 * Encoding details the pages leave open, fixed by this library:
 *   - block scale byte: FP8 E4M3 (bias 7, no infinities, 0x7F unused, largest
 *     finite 448), round-to-nearest-even, clamped to 448;
 *   - tensor scale s_t = A_t / (6 * 448) (binary32), A_t the largest
 *     magnitude of the tensor being quantized (after the Hadamard transform
 *     when one is applied); s_t = 1 when that quotient is 0;
 *   - per block: u = A_b / (6 * s_t), sb = e4m3(u), S = e4m3val(sb) * s_t,
 *     R = 1 / S; per element y = |t| * R, then E2M1 magnitude by RNE (ties to
 *     the even code, y >= 6 saturates) or SR; the sign bit is always copied
 *     (a negative element that rounds to 0 is stored as 0x8);
 *   - SR: element with linear index i in the OUTPUT tensor (row-major in the
 *     stored orientation) draws r = 16 bits of Philox4x32-10 (Salmon et al.,
 *     SC'11) with key (seed low 32, seed high 32) and counter (i/8 low,
 *     i/8 high, stream, 0), word (i%8)/2, low half for even i; stream = 0 for
 *     row blocks, 1 for column blocks, 2 for 16x16 squares; it rounds up iff
 *     r < f * 65536 where f is the fraction of the way from the lower to the
 *     upper neighbouring E2M1 value;
 *   - Hadamard transform: t = (1/4) H16 D x on every aligned group of 16
 *     consecutive elements along the block dimension, H16 the Sylvester
 *     matrix, D = diag(d), d_j = -1 iff bit j of word 0 of Philox4x32-10(key
 *     = hadamard_seed, counter = (0, 0, 3, 0)) is set; evaluated as four
 *     butterfly stages (distance 1, 2, 4, 8; (a, b) -> (a + b, a - b)) then
 *     the multiply by 1/4, in binary32;
 *   - codes are stored two per byte, the even column in bits 3:0.
 *
 * Memory and execution model:
 *   - every pointer is caller-owned DEVICE memory unless stated otherwise;
 *     the library never allocates or frees and keeps no state between calls
 *     (it caches nothing but the device properties it queries);
 *   - every entry point validates its arguments on the host and returns an
 *     error BEFORE launching anything; outputs are then left untouched;
 *   - enumerated arguments and fields are int32_t holding a value of the
 *     enum named beside them, so that any value a caller passes is a defined
 *     input; one outside the enum is refused with NVFP4_ERR_ENUM;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously; NVFP4_ERR_HIP reports a launch failure;
 *   - inputs must be finite; NaN/Inf inputs give unspecified outputs;
 *   - data-pointer alignment: 16 bytes for element arrays and code arrays;
 *     scale arrays and tensor-scale pointers need no alignment beyond their
 *     type.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,        /* a required pointer is NULL */
    NVFP4_ERR_ENUM = 2,        /* an enum argument is out of range */
    NVFP4_ERR_SHAPE = 3,       /* a size is negative, not a multiple of 16 where one is needed, or inconsistent */
    NVFP4_ERR_ALIGN = 4,       /* a pointer or leading dimension violates the alignment rules */
    NVFP4_ERR_UNSUPPORTED = 5, /* a valid but unsupported combination */
    NVFP4_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the size query returned */
    NVFP4_ERR_HIP = 7          /* a HIP launch reported an error */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;

typedef enum {
    NVFP4_ROW_1D = 0,     /* 16 consecutive elements of a row share a scale */
    NVFP4_COL_1D = 1,     /* 16 consecutive elements of a column; output is the transpose */
    NVFP4_ROW_COL_1D = 2, /* both of the above from one read of the input */
    NVFP4_BLK_2D = 3      /* one scale per 16x16 square */
} nvfp4_layout;

typedef enum { NVFP4_RNE = 0, NVFP4_SR = 1 } nvfp4_round;

typedef enum { NVFP4_EPI_NONE = 0, NVFP4_EPI_SWIGLU = 1 } nvfp4_epilogue;

typedef enum { NVFP4_SCALE_1D = 0, NVFP4_SCALE_2D = 1 } nvfp4_scale_mode;

/* A quantized tensor of logical shape rows x cols (stored orientation).
 *   codes:        rows x cols/2 bytes, row-major, even column in bits 3:0.
 *   scales:       SCALE_1D: rows x cols/16 bytes (block of 16 along a row);
 *                 SCALE_2D: rows/16 x cols/16 bytes (16x16 squares).
 *   tensor_scale: one float (grouped GEMM weights: one float per group). */
typedef struct {
    uint8_t* codes;
    uint8_t* scales;
    float* tensor_scale;
    int64_t rows;
    int64_t cols;
    int32_t scale_mode; /* nvfp4_scale_mode */
} nvfp4_tensor;

typedef struct {
    int32_t layout;          /* nvfp4_layout */
    int32_t round;           /* nvfp4_round */
    uint64_t sr_seed;        /* key of the stochastic-rounding draws */
    int32_t hadamard;        /* nonzero: apply the 16-point random Hadamard transform */
    uint64_t hadamard_seed;  /* key of the Hadamard sign draw */
    const float* amax_in;    /* nullable DEVICE pointer: use *amax_in as A_t instead of
                                computing it (the caller vouches that it is the largest
                                magnitude of the tensor being quantized) */
    float* amax_out;         /* nullable DEVICE pointer: receives the A_t used (computed or
                                given), so later calls on the same tensor can pass it as
                                amax_in and skip the amax pass */
} nvfp4_quant_opts;

/* Bytes of workspace nvfp4_quantize needs for this request (0 when amax_in is
 * given). Pure host computation; never fails. */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols, const nvfp4_quant_opts* opts);

/* Quantize x (rows x cols, element dtype `dt`, row stride `ld` elements) to
 * NVFP4 (see the format notes at the top of this file).
 *   ROW_1D:     out[0] is rows x cols, SCALE_1D; cols % 16 == 0.
 *   COL_1D:     out[0] is cols x rows (x transposed), SCALE_1D; rows % 16 == 0.
 *   ROW_COL_1D: out[0] as ROW_1D and out[1] as COL_1D, sharing one A_t;
 *               rows % 16 == 0 and cols % 16 == 0.  With the Hadamard
 *               transform the two outputs quantize two different tensors, x
 *               transformed along rows (out[0]) and x transformed down
 *               columns (out[1]), each with its own A_t: amax_in and
 *               amax_out then point at two floats, out[0]'s first.
 *   BLK_2D:     out[0] is rows x cols, SCALE_2D; both dims % 16 == 0; no
 *               Hadamard transform (UNSUPPORTED).
 * The Hadamard transform runs along the block dimension (along rows for
 * ROW_1D, along columns for COL_1D).  Each out[i] must carry codes, scales
 * and tensor_scale pointers and the rows/cols/scale_mode the layout implies
 * (codes and scales may be NULL when the output has no elements).
 * Requirements: ld >= cols, ld * sizeof(dtype) % 16 == 0, x 16-byte aligned,
 * codes 16-byte aligned; ws_bytes >= nvfp4_quantize_workspace_size(...) and
 * ws 16-byte aligned when that size is nonzero.  rows == 0 or cols == 0 is a
 * no-op that still writes tensor_scale (= 1, or from amax_in).
 * Source: asector.ru page, "NVFP4 и Blackwell"; iitak.ru page, "Детали" and
 * "Как это работает". */
nvfp4_status nvfp4_quantize(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols, int64_t ld,
                            const nvfp4_quant_opts* opts, nvfp4_tensor* out, void* ws,
                            size_t ws_bytes, void* stream);

/* nvfp4_quantize for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, the same results bit for bit.
 * The amax pass keeps its per-workgroup partial maxima in a static device
 * array of the library (512 floats, 2 KiB, one copy per device, held until
 * the process ends) instead of a caller workspace.  That need does not grow
 * with the tensor, so no size is rejected for it.  Nothing is allocated or
 * freed, and nothing needs clearing between calls (every partial a call
 * reads was written by that call).  All calls on one device share the array:
 * calls that overlap in time on one device (on different streams, or from
 * different threads without ordering) race and give unspecified results;
 * calls ordered on one stream do not.  The first call on a device looks the
 * array's address up (hipGetSymbolAddress); NVFP4_ERR_HIP if that fails.
 * Errors otherwise as for nvfp4_quantize. */
nvfp4_status nvfp4_quantize_noalloc(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols, int64_t ld,
                                    const nvfp4_quant_opts* opts, nvfp4_tensor* out, void* stream);

/* Dequantize q into y (q->rows x q->cols in the stored orientation, element
 * dtype `dt`, row stride `ld` elements): y = e2m1(code) * e4m3(scale) *
 * tensor_scale, computed as one binary32 rounding (the first product is
 * exact); BF16 output is the nearest-even BF16 of that value.  Requirements:
 * q->cols % 16 == 0 (and q->rows % 16 == 0 for SCALE_2D), ld >= q->cols,
 * ld * sizeof(dtype) % 16 == 0, y and q->codes 16-byte aligned.
 * Source: iitak.ru page, "Как это работает" (converting back to a more
 * precise format). */
nvfp4_status nvfp4_dequantize(const nvfp4_tensor* q, void* y, int32_t dt /* nvfp4_dtype */, int64_t ld,
                              void* stream);

/* Re-quantize a row-blocked NVFP4 tensor `in` (rows x cols, SCALE_1D) along
 * columns: out (cols x rows, SCALE_1D) receives exactly what nvfp4_quantize
 * with layout COL_1D would produce from the binary32 dequantization of `in`
 * (the values nvfp4_dequantize writes for dtype F32), reading only the codes
 * and scale bytes.  opts: layout must be NVFP4_COL_1D (others return
 * UNSUPPORTED); round, sr_seed, hadamard (along columns), hadamard_seed,
 * amax_in and amax_out as for nvfp4_quantize, where the amax is that of the
 * dequantized tensor (after the transform when hadamard is set).
 * Requirements: rows % 16 == 0, cols % 16 == 0, in->codes and out->codes
 * 16-byte aligned; ws as for nvfp4_quantize (nvfp4_quantize_workspace_size).
 * rows == 0 or cols == 0 only writes out->tensor_scale.  Errors as for
 * nvfp4_quantize.
 * Source: iitak.ru page, "Как это работает" (row blocks of the forward
 * tensor re-formed along columns for the backward pass). */
nvfp4_status nvfp4_requantize(const nvfp4_tensor* in, const nvfp4_quant_opts* opts, nvfp4_tensor* out,
                              void* ws, size_t ws_bytes, void* stream);

/* C = A * B^T for A (M x K) and B (N x K) NVFP4 tensors, accumulated in
 * binary32 over exactly dequantized products; C (M x N, row stride ldc
 * elements, dtype c_dt) = (s_A * s_B) * sum_k (v_A sb_A)(v_B sb_B).
 * Each operand may be SCALE_1D or SCALE_2D.  K % 16 == 0, M, N >= 0,
 * ldc >= N, C 16-byte aligned, codes 16-byte aligned.
 *   EPI_NONE:   as above.
 *   EPI_SWIGLU: N = 2F with F % 16 == 0; gate = columns [0, F), up = columns
 *               [F, 2F) of A * B^T; C (M x F, ldc >= F) = gate *
 *               sigmoid(gate) * up, and c_dt must be BF16 (else
 *               UNSUPPORTED).  The grouped GEMM offers the same epilogue
 *               with the largest |C| written to amax_out.
 * Workspace (optional): with ws 16-byte aligned and ws_bytes >=
 * nvfp4_gemm_workspace_size(A, B, c_dt, ep) > 0, a last round of 256 x 256
 * output tiles that would leave compute units idle is computed in parts
 * along K, whose binary32 sums are added in a fixed order (and, for BF16
 * output, rounded once); ws NULL or smaller: no split.  The two give the same accuracy, not always the same
 * last bits; each is deterministic on a given device (the split depends on
 * its compute-unit count).  ws is scratch for this call only: calls that
 * overlap must not share it.
 * Source: asector.ru page, "NVFP4 и Blackwell" (scaled compute with
 * high-precision accumulation); iitak.ru page, "Детали" (the expert layers
 * whose feed-forward the SwiGLU epilogue closes). */
nvfp4_status nvfp4_gemm(const nvfp4_tensor* A, const nvfp4_tensor* B, void* C, int32_t c_dt /* nvfp4_dtype */,
                        int64_t ldc, int32_t ep /* nvfp4_epilogue */, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace with which nvfp4_gemm splits its last round of tiles on
 * the current device: nonzero only without an epilogue (FP32 or BF16
 * output), K % 512 == 0 and a tile count that leaves a partial last round
 * with enough idle compute units; 0 also for invalid arguments or when the
 * device cannot be queried.  At most 8 parts of 256 KiB per tile of that
 * round. */
size_t nvfp4_gemm_workspace_size(const nvfp4_tensor* A, const nvfp4_tensor* B, int32_t c_dt /* nvfp4_dtype */,
                                 int32_t ep /* nvfp4_epilogue */);

/* Grouped (mixture-of-experts) GEMM.  A is sum_g M_g x K with one tensor
 * scale; rows offsets[g] .. offsets[g+1]-1 belong to group g (offsets: DEVICE
 * int64[G+1], nondecreasing, offsets[0] = 0, offsets[G] = A->rows).  B stacks
 * the G weight matrices, B->rows = G * N_g, B->tensor_scale points at G
 * floats; group g uses rows g*N_g .. (g+1)*N_g-1 of B.
 *   EPI_NONE:   C rows of group g = A_g * B_g^T, C is A->rows x N_g.
 *   EPI_SWIGLU: N_g = 2F; gate = columns [0, F), up = columns [F, 2F) of
 *               A_g * B_g^T; C = gate * sigmoid(gate) * up, A->rows x F, and
 *               c_dt must be BF16.  If amax_out (DEVICE float) is non-NULL it
 *               receives the largest |C| as stored (for a following quantize
 *               with amax_in).
 * The host never reads the device offsets: it sizes the launch from
 * sum_g M_g = A->rows and G.  A must be SCALE_1D.  Requirements as for
 * nvfp4_gemm; B->rows % G == 0; for SCALE_2D B, N_g % 16 == 0; for SwiGLU
 * N_g % 2 == 0 and F % 16 == 0.  Offsets that break the rules above give
 * unspecified results but no out-of-bounds access (group ranges are clamped
 * to [0, A->rows]).  No workspace is needed; ws/ws_bytes are reserved and may
 * be NULL/0.
 * Source: iitak.ru page, "Детали" (NVFP4 in the expert layers' forward pass)
 * and "Но" (experts spread over GPUs). */
nvfp4_status nvfp4_grouped_gemm(int32_t G, const nvfp4_tensor* A, const int64_t* offsets,
                                const nvfp4_tensor* B, void* C,
                                int32_t c_dt /* nvfp4_dtype */, int64_t ldc, int32_t ep /* nvfp4_epilogue */, float* amax_out,
                                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * MX formats (OCP Microscaling).  The pages name MXFP8 (the backward-pass
 * format at Thinking Machines: iitak.ru page, "Как это работает"), MXFP4 (the
 * Open Compute Project format NVFP4 is compared with: asector.ru page,
 * "Перспективы и дальнейшие направления исследований") and an 8.25-bit
 * transit format for expert outputs (iitak.ru page, "Но"), without defining
 * them.  This library reads
 * them as OCP Microscaling:
 *   - 32 consecutive elements along the block dimension share an E8M0 scale
 *     byte b = s + 127 (value 2^s), s = floor(log2(max|V|)) - emax, emax = 8
 *     for E4M3 elements and 2 for E2M1, clamped to [-127, 127]; s = -127 for
 *     an all-zero block;
 *   - element code: y = fl(|V| * 2^-s), rounded onto E4M3 (as the NVFP4 scale
 *     byte: bias 7, largest 448 = 0x7E) or E2M1 to nearest-even, or
 *     stochastically (round up iff r < f * 65536 with r the 16-bit Philox
 *     draw of the element, as for NVFP4, stream 4 for ROW_1D and 5 for
 *     COL_1D); y beyond the largest value saturates (448 or 6); the sign is
 *     copied (bit 7 for E4M3, bit 3 for E2M1);
 *   - E4M3 with 32-element blocks costs 8 + 8/32 = 8.25 bits per element.
 * ---------------------------------------------------------------------- */
typedef enum { NVFP4_MX_E4M3 = 0, NVFP4_MX_E2M1 = 1 } nvfp4_mx_elem;

/* An MX tensor of logical shape rows x cols (stored orientation).
 *   codes:  E4M3: rows x cols bytes; E2M1: rows x cols/2 bytes, even column
 *           in bits 3:0; row-major.
 *   scales: rows x cols/32 E8M0 bytes (2^(byte - 127); byte 0xFF is not
 *           produced and dequantizes to an unspecified value). */
typedef struct {
    uint8_t* codes;
    uint8_t* scales;
    int64_t rows;
    int64_t cols;
    int32_t elem; /* nvfp4_mx_elem */
} nvfp4_mx_tensor;

/* MX-quantize x (rows x cols, dtype dt, row stride ld elements) into out,
 * whose elem field selects the element format.
 *   ROW_1D: blocks along rows; out is rows x cols; cols % 32 == 0.
 *   COL_1D: blocks along columns; out is cols x rows (x transposed);
 *           rows % 32 == 0.
 *   other layouts return NVFP4_ERR_UNSUPPORTED.
 * No tensor scale and no workspace.  Requirements: ld >= cols,
 * ld * sizeof(dtype) % 16 == 0, x and out->codes 16-byte aligned; out->rows
 * and out->cols as the layout implies.  rows == 0 or cols == 0 is a no-op.
 * Errors as for nvfp4_quantize. */
nvfp4_status nvfp4_mx_quantize(const void* x, int32_t dt /* nvfp4_dtype */, int64_t rows, int64_t cols, int64_t ld,
                               int32_t layout /* nvfp4_layout */, int32_t round /* nvfp4_round */, uint64_t sr_seed,
                               nvfp4_mx_tensor* out, void* stream);

/* y = value(code) * 2^(scale byte - 127) as one binary32 rounding (exact
 * unless the result leaves the binary32 normal range); BF16 output is the
 * nearest-even BF16 of that binary32 value.  y is q->rows x q->cols, row
 * stride ld elements.  Requirements: q->cols % 32 == 0, ld >= q->cols,
 * ld * sizeof(dtype) % 16 == 0, y and q->codes 16-byte aligned. */
nvfp4_status nvfp4_mx_dequantize(const nvfp4_mx_tensor* q, void* y, int32_t dt /* nvfp4_dtype */, int64_t ld,
                                 void* stream);

/* How nvfp4_mx_gemm accumulates.
 *   NATIVE: gfx950's scaled matrix cores take the codes and scale bytes as
 *           they are (the fastest path).  The OCP Microscaling definition
 *           leaves the internal precision of a block dot product to the
 *           implementation; this hardware sums the 64 products of a K step
 *           exactly for E2M1 operands, but for E4M3 operands keeps about 13
 *           significant bits relative to the step's largest product (errors
 *           up to ~2^-12 of it, measured), so E4M3 results do NOT meet the
 *           1e-5 * sum |a b| accuracy of nvfp4_gemm.
 *   EXACT:  every element is converted exactly to BF16 times a power of two
 *           relative to its row's largest block scale, and the BF16 matrix
 *           cores form every product exactly and sum in binary32, as
 *           nvfp4_gemm does: |C - sum of exact products| within
 *           1e-5 * sum |a b| (+ half a BF16 ulp for BF16 output), at about
 *           the FP16 matrix-core rate.  Exact products need the rescaled
 *           elements and their products in the normal ranges of BF16 and
 *           binary32: it suffices that in every row of A and of B the nonzero
 *           blocks' scales lie within 2^54 of the row's largest, and that C
 *           stays within binary32's range. */
typedef enum { NVFP4_MX_ACC_NATIVE = 0, NVFP4_MX_ACC_EXACT = 1 } nvfp4_mx_accum;

/* C = A * B^T for MX tensors A (M x K) and B (N x K) of the same element
 * format: C[m][n] = sum over K of (v_A 2^s_A)(v_B 2^s_B), accumulated as
 * `accum` (nvfp4_mx_accum) selects, written as F32 or BF16 (nearest even) to
 * C (M x N, row stride ldc elements).
 * Requirements: K % 64 == 0 (K % 32 != 0 is ERR_SHAPE, K % 64 == 32 is
 * ERR_UNSUPPORTED), code bytes per row (K for E4M3, K/2 for E2M1) below
 * 2^24 (else ERR_UNSUPPORTED), A->elem == B->elem (else ERR_UNSUPPORTED), ldc >= N,
 * codes 16-byte aligned, scales 2-byte aligned, C aligned to its element.
 * Source: asector.ru page, "NVFP4 и Blackwell" (block-scaled tensor-core
 * compute); iitak.ru page, "Как это работает" (MXFP8 in the backward pass). */
nvfp4_status nvfp4_mx_gemm(const nvfp4_mx_tensor* A, const nvfp4_mx_tensor* B, void* C, int32_t c_dt /* nvfp4_dtype */,
                           int64_t ldc, int32_t accum, void* ws, size_t ws_bytes, void* stream);

/* Workspace of nvfp4_mx_gemm (optional, as for nvfp4_gemm): with ws 16-byte
 * aligned and ws_bytes >= nvfp4_mx_gemm_workspace_size(A, B, c_dt, accum) >
 * 0, a last round of 256 x 256 tiles that would leave compute units idle is
 * computed in parts along K (whole 1024-element units) whose binary32 sums
 * are added in a fixed order (both accumulation modes; exact: each part's
 * sums scaled as the whole tile's; BF16 output: rounded once); nonzero only
 * for K % 1024 == 0 and such a last round on the current device, where the
 * library's estimate of the split's saving exceeds its cost (parts written
 * and summed); 0 also for invalid arguments or when the device cannot be
 * queried. */
size_t nvfp4_mx_gemm_workspace_size(const nvfp4_mx_tensor* A, const nvfp4_mx_tensor* B, int32_t c_dt /* nvfp4_dtype */,
                                    int32_t accum);

/* Static description of a status code. */
const char* nvfp4_status_string(int32_t s /* nvfp4_status */);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t nvfp4_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4_H */
