// NVFP4 quantize, tensor-amax and dequantize kernels for gfx950.
//
// Quantization with a 16-element block multiplier and a per-tensor scale
// ("Nvidia добивается успеха с 4-битным форматом NVFP4", asector.ru, section
// "NVFP4 и Blackwell: интеграция архитектуры и формата"; "Thinking Machines
// ускорила обучение Inkling 2 Small 4-битными числами", iitak.ru, section
// "Детали"), in three block layouts: along rows, along columns (the flipped
// tables of the backward pass) and 16x16 squares (iitak.ru page, "Как это
// работает"), with an optional 16-point random Hadamard transform (asector.ru
// page, "Эксперименты и сравнение с FP8").
//
// All of these are HBM-bound streaming kernels whose second limit is VALU
// issue (Philox dominates under stochastic rounding).  Shared structure:
//   - 256-thread workgroups (four wave64s); grid dimension x runs over column
//     groups, so workgroups dispatched together sweep contiguous stretches of
//     each row (this alone is worth ~25% of HBM throughput against a
//     row-group-first order); dimension y runs over row groups (the row and
//     dequantize kernels loop over row groups beyond 65535);
//   - 16-byte loads whose lanes cover contiguous spans, and every 128-byte
//     output line written by one workgroup (or by workgroups dispatched
//     together);
//   - the tensor amax is a separate streaming pass writing at most
//     kMaxPartials per-workgroup maxima, which every consumer wave reduces
//     in its prologue (issued after the wave's first loads, no barrier),
//     unless the caller supplies the amax;
//   - column blocks go through an LDS transpose: a 256-row x 128-byte tile is
//     loaded with full-row 16-byte loads, written to LDS with a per-row-band
//     XOR swizzle, and read back as 16-row x 8-byte column strips, so every
//     thread ends up with whole column blocks and each 128-byte line of the
//     transposed output comes from 16 lanes of one wave;
//   - a 16-element row block lives in a lane pair (quad for fp32 input); the
//     lanes join their maxima with lane exchanges and split the block-scale
//     arithmetic between rows;
//   - nearest-even encoding uses the gfx950 FP4 pack instruction on the
//     already-scaled values (scale operand 1.0), two codes per instruction;
//     stochastic rounding uses the gfx950 SR convert, one code per
//     instruction, with the value pre-rounded so that the instruction's
//     decision is exactly "draw < fraction" (see encode()).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

// ============================================================ amax
// A_t for the calling wave: n == 0 means src[0] is A_t itself, otherwise the
// maximum of the n partials src[0..n) (n <= kMaxPartials).  Every wave reduces
// the partials on its own (eight L2-resident loads per lane, issued together
// from clamped indices, then lane exchanges), so no barrier is needed and the
// caller's own loads can be in flight meanwhile.
__device__ __forceinline__ float tensor_amax_of(const float* __restrict__ src, int n) {
    if (n == 0) return src[0];
    constexpr int PER_LANE = (int)(kMaxPartials / 64);
    const int lane = threadIdx.x & 63;
    float p[PER_LANE];
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) p[k] = src[min(lane + 64 * k, n - 1)];
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) a = fmaxf(a, p[k]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    return a;
}

template <int NT = 256>
__device__ __forceinline__ void store_partial(float a, float* __restrict__ partial) {
    __shared__ float red[NT / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
#pragma unroll
        for (int k = 1; k < NT / 64; ++k) m = fmaxf(m, red[k]);
        partial[blockIdx.y * gridDim.x + blockIdx.x] = m;
    }
}

// Element e of a raw 16-byte chunk (bf16 pairs or fp32).
template <typename T>
__device__ __forceinline__ float chunk_elem(const uint4& q, int e) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t w = (e >> 1) == 0 ? q.x : (e >> 1) == 1 ? q.y : (e >> 1) == 2 ? q.z : q.w;
        return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    } else {
        return __uint_as_float(e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w);
    }
}

// 16-byte chunk j of row `row` as binary32 (8 bf16 or 4 fp32 values).
template <typename T>
__device__ __forceinline__ void load_chunk(const T* __restrict__ row, int64_t j, float v[8]) {
    if constexpr (sizeof(T) == 2) {
        load8(reinterpret_cast<const uint16_t*>(row) + j * 8, v);
    } else {
        float4 q = *reinterpret_cast<const float4*>(row + j * 4);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
}

// Partial maxima of |x| (no transform).  Rows by, by + gy, ...; in each row
// the 16-byte chunks bx*256*U + tid + 256*u + k*(gx*256*U), U = 8 per thread
// per iteration (128 bytes in flight per thread keeps enough requests
// outstanding with only kMaxPartials workgroups).  A contiguous tensor is
// passed as one long row.
template <typename T>
__global__ void __launch_bounds__(256) k_amax_plain(const T* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld,
                                                    float* __restrict__ partial) {
    constexpr int CH = 16 / sizeof(T);
    constexpr int U = 8;
    const int64_t nfull = cols / CH;  // chunks wholly inside a row
    const int64_t nch = (cols + CH - 1) / CH;
    const int64_t step = (int64_t)gridDim.x * 256 * U;
    float a = 0.0f;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const T* row = x + r * ld;
        int64_t j0 = (int64_t)blockIdx.x * 256 * U + threadIdx.x;
        // all U chunks in range: unconditional loads, issued back to back
        for (; j0 + 256 * (U - 1) < nfull; j0 += step) {
            float v[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u) load_chunk(row, j0 + 256 * u, v[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < CH; ++e) a = fmaxf(a, fabsf(v[u][e]));
        }
        // the rest, chunk by chunk
        for (; j0 < nch; j0 += step) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t j = j0 + 256 * u;
                if (j >= nch) continue;
                float v[8];
                load_chunk(row, j, v);
                const int64_t valid = cols - j * CH;
#pragma unroll
                for (int e = 0; e < CH; ++e)
                    if (e < valid) a = fmaxf(a, fabsf(v[e]));
            }
        }
    }
    store_partial(a, partial);
}

// Partial maxima of |H16 D x| with the transform along rows (16 consecutive
// columns; cols % 16 == 0): two 16-element groups per thread per row.
template <typename T>
__global__ void __launch_bounds__(256) k_amax_hadamard_rows(const T* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ld,
                                                            uint32_t sign_mask,
                                                            float* __restrict__ partial) {
    const int64_t nb = cols / 16;
    float a = 0.0f;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        for (int64_t b0 = (int64_t)blockIdx.x * 512 + threadIdx.x; b0 < nb; b0 += (int64_t)gridDim.x * 512) {
            float v[2][16];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t b = b0 + 256 * u;
                if (b < nb) {
                    load8(x + r * ld + b * 16, v[u]);
                    load8(x + r * ld + b * 16 + 8, v[u] + 8);
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) v[u][e] = 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) a = fmaxf(a, hadamard16_absmax(v[u], sign_mask));
        }
    }
    store_partial(a, partial);
}

// Partial maxima with the transform down columns (16 consecutive rows;
// rows % 16 == 0).  A thread owns a 16-row x 16-byte patch, kept as the 16
// loaded chunks and unpacked one column at a time (BF16: 64 registers for the
// chunks instead of 128 for the unpacked values), in 512-thread workgroups:
// the grid is capped at kMaxPartials workgroups, so the threads per
// workgroup set how many loads are in flight.
constexpr int kAmaxColsThreads = 512;

template <typename T>
__global__ void __launch_bounds__(kAmaxColsThreads) k_amax_hadamard_cols(const T* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ld,
                                                            uint32_t sign_mask,
                                                            float* __restrict__ partial) {
    constexpr int CH = 16 / sizeof(T), NT = kAmaxColsThreads;
    const int64_t nch = (cols + CH - 1) / CH;
    const int64_t nrb = rows / 16;
    float a = 0.0f;
    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
        for (int64_t j = (int64_t)blockIdx.x * NT + threadIdx.x; j < nch; j += (int64_t)gridDim.x * NT) {
            uint4 raw[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) raw[i] = *reinterpret_cast<const uint4*>(x + (rb * 16 + i) * ld + j * CH);
            const int64_t valid = cols - j * CH;
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                float col[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) col[i] = chunk_elem<T>(raw[i], e);
                const float t = hadamard16_absmax(col, sign_mask);
                if (e < valid) a = fmaxf(a, t);
            }
        }
    }
    store_partial<NT>(a, partial);
}

// tensor_scale (and amax_out) of an empty tensor: no element kernel runs.
__global__ void k_write_tensor_scale(const float* amax_in, float* ts0, float* ts1, float* amax_out) {
    float a = amax_in ? amax_in[0] : 0.0f;
    float st = tensor_scale_of(a);
    if (ts0) ts0[0] = st;
    if (ts1) ts1[0] = st;
    if (amax_out) amax_out[0] = a;
}

// Shared prologue: reduce A_t, derive s_t, fill the workgroup's table of
// block multipliers (one entry per E4M3 byte), and let workgroup 0 publish s_t
// and A_t.  Every thread of the (256-thread) workgroup must call it: it ends
// with a barrier.
struct TensorScale {
    float st, six_st;
    const float* rtab;  // 128 block multipliers in LDS
};

__device__ __forceinline__ TensorScale prologue(const float* amax_src, int n_partials, float* ts0,
                                                float* ts1, float* amax_out) {
    __shared__ float rtab[128];
    const float a = tensor_amax_of(amax_src, n_partials);
    TensorScale t;
    t.st = tensor_scale_of(a);
    t.six_st = 6.0f * t.st;
    if (threadIdx.x < 128) rtab[threadIdx.x] = block_multiplier(threadIdx.x, t.st);
    __syncthreads();
    t.rtab = rtab;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        if (ts0) ts0[0] = t.st;
        if (ts1) ts1[0] = t.st;
        if (amax_out) amax_out[0] = a;
    }
    return t;
}

// ============================================================ shared pieces
// The Hadamard transform of a block split over a lane pair: stages 1, 2, 4 run
// in each lane; the distance-8 stage pairs element j of the even lane with
// element j of the odd lane, computed as (even + odd) on the even lane and
// (even - odd) on the odd lane -- the same operations on the same operands as
// the sequential butterfly.
__device__ __forceinline__ void hadamard8_pair(float v[8], uint32_t sign_mask, bool odd) {
    const uint32_t m = odd ? (sign_mask >> 8) : sign_mask;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if ((m >> j) & 1u) v[j] = -v[j];
#pragma unroll
    for (int hh = 1; hh < 8; hh <<= 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j & hh) continue;
            float a = v[j], b = v[j + hh];
            v[j] = a + b;
            v[j + hh] = a - b;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float p = lane_xor1(v[j]);
        v[j] = odd ? (p - v[j]) : (v[j] + p);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.25f * v[j];
}

// Lane-pair block scales for two rows (r, r+1) whose 16-element blocks are
// split 8 + 8 between lanes 2k (even) and 2k+1 (odd): both lanes join both
// rows' maxima, the even lane derives row r's multiplier and the odd lane row
// r+1's, and one exchange hands each lane both.  a0, a1 return the joined
// block maxima.
__device__ __forceinline__ void pair_block_scales(float& a0, float& a1, bool odd, const TensorScale& ts,
                                                  BlockScale& b0, BlockScale& b1) {
    a0 = fmaxf(a0, lane_xor1(a0));
    a1 = fmaxf(a1, lane_xor1(a1));
    const BlockScale mine = block_scale(odd ? a1 : a0, ts.six_st, ts.rtab);
    BlockScale other;
    other.R = lane_xor1(mine.R);
    other.byte = lane_xor1(mine.byte);
    b0 = odd ? other : mine;
    b1 = odd ? mine : other;
}

// ============================================================ ROW_1D
// Every lane holds 8 consecutive elements of a row (one 16-byte load for bf16,
// two for fp32); lanes 2k and 2k+1 hold the two halves of one 16-element block.
// Wave w owns rows 8 * rg + 2w, +1 of row group rg and 512 columns from
// 512 * blockIdx.x; a wave-wide load reads 1 KiB (bf16) of one row.
template <typename T, bool SR, bool RHT>
__global__ void __launch_bounds__(256) k_quant_row(const T* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld,
                                                   const float* __restrict__ amax_src, int n_part,
                                                   uint64_t seed, uint32_t sign_mask,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales,
                                                   float* __restrict__ ts_out, float* amax_out) {
    const int lane = threadIdx.x & 63;
    const bool odd = lane & 1;
    const int64_t c = (int64_t)blockIdx.x * 512 + 8 * lane;
    const bool col_ok = c < cols;  // cols % 16 == 0: both lanes of a pair agree
    // Lanes past the last column and rows past the last row read a clamped
    // in-range chunk whose results are never stored, so the loads carry no
    // branch and issue together.
    const int64_t cl = col_ok ? c : cols - 8;
    const int64_t nrg = (rows + 7) / 8;
    float v[2][8];
    auto load_group = [&](int64_t rg) {
        const int64_t r = rg * 8 + 2 * (threadIdx.x >> 6);
#pragma unroll
        for (int k = 0; k < 2; ++k) load8(x + (r + k < rows ? r + k : rows - 1) * ld + cl, v[k]);
    };
    int64_t rg = blockIdx.y;  // < nrg: grid y is at most the row-group count
    load_group(rg);
    const TensorScale ts = prologue(amax_src, n_part, ts_out, nullptr, amax_out);
    for (;;) {
        const int64_t r = rg * 8 + 2 * (threadIdx.x >> 6);
        if (RHT) {
            hadamard8_pair(v[0], sign_mask, odd);
            hadamard8_pair(v[1], sign_mask, odd);
        }
        float a[2] = {0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) a[k] = fmaxf(a[k], fabsf(v[k][e]));
        BlockScale bs[2];
        pair_block_scales(a[0], a[1], odd, ts, bs[0], bs[1]);
        if (col_ok) {
            uint32_t wd[2][4];
            if (SR) philox_words2(seed, kStreamRow, (uint64_t)(r * cols + c), (uint64_t)((r + 1) * cols + c), wd[0], wd[1]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (r + k >= rows) break;
                uint32_t w[1];
                encode<SR, 8, sizeof(T) == 2 && !RHT>(v[k], bs[k], a[k], wd[k], w);
                // codes go out non-temporally (a wave's store is two whole
                // 128-byte lines): they then leave the caches to the input,
                // which further quantizations of the same tensor re-read.
                // Measured on 8192^2 BF16: six quantizations and two
                // dequantizations of one tensor 342 -> 329 us, this kernel
                // alone 29.5 -> 30.8 us.
                __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(codes + (r + k) * (cols / 2) + c / 2));
                if (odd == (k == 1)) scales[(r + k) * (cols / 16) + c / 16] = (uint8_t)bs[k].byte;
            }
        }
        rg += gridDim.y;
        if (rg >= nrg) break;
        load_group(rg);
    }
}

// ============================================================ LDS transpose tile
// COL_1D and ROW_COL_1D.  Workgroup (x, y) owns the tile of 256 rows from
// 256 * y and 128 bytes of each row (TWC = 64 bf16 or 32 fp32 columns) from
// column TWC * x.
//   load: thread t reads 16-byte chunk t % 8 of tile rows t / 8 + 32 k
//     (k = 0..7): each wave-wide load covers 8 rows x 128 bytes.  The chunk's
//     two 8-byte units land in LDS at unit (2 ch + h) ^ (band % 16) of the row
//     (band = row / 16; rows padded to 136 bytes), so the column reads below
//     spread over the banks;
//   row blocks (ROW_COL): straight from the loaded chunks, a 16-element block
//     spanning LPB = 2 (bf16) or 4 (fp32) lanes, as in the row kernel;
//   column blocks: thread t takes row band t % 16 and 8-byte unit t / 16: 16
//     LDS reads give it 16 rows x UE columns (UE = 4 bf16 or 2 fp32), i.e. UE
//     complete column blocks.  The 16 lanes that share a unit write the 16
//     consecutive 8-byte code groups (one 128-byte line) of each column.
template <typename T>
struct ColTile {
    static constexpr int CH = 16 / sizeof(T);    // elements per 16-byte chunk
    static constexpr int TWC = 128 / sizeof(T);  // tile width in columns
    static constexpr int UE = 8 / sizeof(T);     // elements per 8-byte unit
    static constexpr int LPB = 16 / CH;          // lanes per 16-element row block
    static constexpr int STRIDE = 136;           // LDS bytes per tile row
};

// Element e of a raw 8-byte unit.
template <typename T>
__device__ __forceinline__ float unit_elem(const uint2& q, int e) {
    if constexpr (sizeof(T) == 2) {
        const uint32_t w = (e >> 1) == 0 ? q.x : q.y;
        return (e & 1) ? __uint_as_float(w & 0xFFFF0000u) : __uint_as_float(w << 16);
    } else {
        return __uint_as_float(e == 0 ? q.x : q.y);
    }
}

// Row blocks of the 8 loaded chunks (ROW_COL): rows R0 + t/8 + 32 k, columns
// gc .. gc + CH - 1.  cols % 16 == 0 and rows % 16 == 0, so the LPB lanes of a
// block agree on validity.
template <typename T, bool SR>
__device__ __forceinline__ void tile_row_blocks(const uint4 (&raw)[8], int64_t R0, int lr0, int64_t gc,
                                                int64_t rows, int64_t cols, const TensorScale& ts,
                                                uint64_t seed, uint8_t* __restrict__ rcodes,
                                                uint8_t* __restrict__ rscales) {
    constexpr int CH = ColTile<T>::CH, LPB = ColTile<T>::LPB;
    const int lane = threadIdx.x & 63;
    const int q = lane % LPB;
    const bool col_ok = gc < cols;
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < CH; ++e) m = fmaxf(m, fabsf(chunk_elem<T>(raw[k], e)));
        m = fmaxf(m, lane_xor1(m));
        if (LPB == 4) m = fmaxf(m, lane_xor2(m));
        a[k] = m;
    }
    // lane q of a block derives the multipliers of rows k = q, q + LPB, ...;
    // the lanes then exchange them
    BlockScale bs[8];
#pragma unroll
    for (int i0 = 0; i0 < 8; i0 += LPB) {
        float mine_a = a[i0];
#pragma unroll
        for (int k = 1; k < LPB; ++k) mine_a = (q == k) ? a[i0 + k] : mine_a;
        const BlockScale mine = block_scale(mine_a, ts.six_st, ts.rtab);
#pragma unroll
        for (int k = 0; k < LPB; ++k) {
            bs[i0 + k].R = group_lane<LPB>(mine.R, k);
            bs[i0 + k].byte = group_lane<LPB>(mine.byte, k);
        }
    }
    // the lane's output addresses and draw index for row R0 + lr0, stepped by
    // wave-uniform multiples of 32 rows (no per-row 64-bit products)
    const int64_t rl0 = R0 + lr0;
    uint8_t* const dst0 = rcodes + rl0 * (cols / 2) + gc / 2;
    uint8_t* const sdst0 = rscales + rl0 * (cols / 16) + gc / 16;
    const uint64_t idx0 = (uint64_t)((rl0 * cols + gc) & ~(int64_t)7);  // + 32 k cols keeps the & ~7
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        const int64_t r = rl0 + 32 * k;  // rows r and r + 32
        if (!col_ok || r >= rows) continue;
        uint32_t wd[2][4];
        if (SR) {
            philox_words2(seed, kStreamRow, idx0 + (uint64_t)(32 * k) * cols, idx0 + (uint64_t)(32 * k + 32) * cols,
                          wd[0], wd[1]);
            if (CH == 4 && (gc & 4)) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    wd[h][0] = wd[h][2];
                    wd[h][1] = wd[h][3];
                }
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t rr = r + 32 * h;
            if (rr >= rows) continue;
            float v[8];
#pragma unroll
            for (int e = 0; e < CH; ++e) v[e] = chunk_elem<T>(raw[k + h], e);
#pragma unroll
            for (int e = CH; e < 8; ++e) v[e] = 0.0f;
            uint32_t w[1];
            encode<SR, 8, sizeof(T) == 2>(v, bs[k + h], a[k + h], wd[h], w);
            uint8_t* dst = dst0 + (int64_t)(32 * (k + h)) * (cols / 2);
            // plain stores (not non-temporal as in the row kernel): these
            // 32-byte pieces of a row's line are completed by other
            // workgroups of the same XCD, and only the L2 combines them
            // (written past it, 8192^2 BF16: the stochastic-rounding
            // instance wrote 108 MiB instead of 81 for 72 MiB of outputs,
            // and the round-to-nearest instance took 63 us instead of 49)
            if (CH == 8) *reinterpret_cast<uint32_t*>(dst) = w[0];
            else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[0];
            if (q == (k + h) % LPB) sdst0[(int64_t)(32 * (k + h)) * (cols / 16)] = (uint8_t)bs[k + h].byte;
        }
    }
}

// Sign-flip words of the BF16 transform path below: bit 31 of sflip[i] is
// bit i of sign_mask.
__device__ __forceinline__ void sign_flips16(uint32_t sign_mask, uint32_t (&sflip)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sflip[i] = ((sign_mask >> i) & 1u) << 31;
}

// Column block e of a 16-row unit q (row i's 8 bytes in q[i]: UE columns):
// codes into w[0..1] (rows in order), the block scale returned.  idx is the
// output index of the block's first element (its draws).  BF16 with the
// transform: row i's sign flip rides on the unpack (adding 2^31 flips the top
// bit; sflip from sign_flips16), and the multiply by 1/4 on the block
// multiplier (encode_quarter16).
template <typename T, bool SR, bool RHT>
__device__ __forceinline__ BlockScale col_unit_block(const uint2 (&q)[16], int e, const uint32_t (&sflip)[16],
                                                     uint32_t sign_mask, const TensorScale& ts, uint64_t seed,
                                                     uint64_t idx, uint32_t (&w)[2]) {
    constexpr bool QUARTER = RHT && sizeof(T) == 2;
    float col[16];
    if constexpr (QUARTER) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t wd2 = (e >> 1) == 0 ? q[i].x : q[i].y;
            col[i] = __uint_as_float((e & 1) ? ((wd2 & 0xFFFF0000u) ^ sflip[i]) : ((wd2 << 16) + sflip[i]));
        }
        hadamard16_sums(col);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) col[i] = unit_elem<T>(q[i], e);
        if (RHT) hadamard16(col, sign_mask);
    }
    const float ab = QUARTER ? 0.25f * absmax16(col) : absmax16(col);
    const BlockScale bs = block_scale(ab, ts.six_st, ts.rtab);
    uint32_t wd[8];
    if (SR) philox_words16(seed, kStreamCol, idx, wd);
    if constexpr (QUARTER) encode_quarter16<SR>(col, bs, ab, wd, w);
    else encode<SR, 16, sizeof(T) == 2 && !RHT>(col, bs, ab, wd, w);
    return bs;
}

// Column blocks of a staged tile (after the barrier): thread t takes row band
// t % 16 and 8-byte unit t / 16 (16 rows x UE columns), i.e. UE whole column
// blocks of the transposed output.
template <typename T, bool SR, bool RHT>
__device__ __forceinline__ void tile_col_blocks(const uint8_t* tile, int64_t R0, int64_t C0, int64_t rows,
                                                int64_t cols, const TensorScale& ts, uint64_t seed,
                                                uint32_t sign_mask, uint8_t* __restrict__ ccodes,
                                                uint8_t* __restrict__ cscales) {
    constexpr int UE = ColTile<T>::UE, STRIDE = ColTile<T>::STRIDE;
    const int t = threadIdx.x;
    const int rb = t & 15, u = t >> 4;
    const int64_t r0 = R0 + 16 * rb;
    if (r0 >= rows) return;  // rows % 16 == 0: a band is wholly inside or outside (no barrier follows)
    uint2 q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        q[i] = *reinterpret_cast<const uint2*>(tile + (16 * rb + i) * STRIDE + 8 * (u ^ rb));
    uint32_t sflip[16];
    sign_flips16(sign_mask, sflip);
    // the lane's output addresses and draw index for column C0 + UE u, stepped
    // by wave-uniform multiples of a column
    const int64_t cl0 = C0 + UE * u;
    uint8_t* const cdst0 = ccodes + cl0 * (rows / 2) + r0 / 2;
    uint8_t* const csdst0 = cscales + cl0 * (rows / 16) + r0 / 16;
    const uint64_t cidx0 = (uint64_t)(cl0 * rows + r0);
#pragma unroll
    for (int e = 0; e < UE; ++e) {
        const int64_t c = cl0 + e;
        if (c >= cols) continue;  // (not break: the loop must unroll fully)
        uint32_t w[2];
        const BlockScale bs = col_unit_block<T, SR, RHT>(q, e, sflip, sign_mask, ts, seed, cidx0 + (uint64_t)e * rows, w);
        // non-temporal as in the row kernel: the 16 lanes of a column write
        // one whole 128-byte line
        typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
        const v2u_t cw = {w[0], w[1]};
        __builtin_nontemporal_store(cw, reinterpret_cast<v2u_t*>(cdst0 + (int64_t)e * (rows / 2)));
        csdst0[(int64_t)e * (rows / 16)] = (uint8_t)bs.byte;
    }
}

// At least three waves per SIMD: the fused stochastic-rounding instance must
// stay within 168 VGPRs.
template <typename T, bool DO_ROW, bool SR, bool RHT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) k_quant_colt(const T* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld,
                                                    const float* __restrict__ amax_src, int n_part,
                                                    uint64_t seed, uint32_t sign_mask,
                                                    uint8_t* __restrict__ rcodes,
                                                    uint8_t* __restrict__ rscales,
                                                    float* __restrict__ rts,
                                                    uint8_t* __restrict__ ccodes,
                                                    uint8_t* __restrict__ cscales,
                                                    float* __restrict__ cts, float* amax_out,
                                                    int xcd_group) {
    constexpr int CH = ColTile<T>::CH, TWC = ColTile<T>::TWC, STRIDE = ColTile<T>::STRIDE;
    __shared__ __attribute__((aligned(16))) uint8_t tile[256 * STRIDE];
    const int t = threadIdx.x;
    const TileXY tl = xcd_tile_pairs(xcd_group);
    const int64_t R0 = tl.y * 256, C0 = tl.x * TWC;

    // ---- load 256 rows x 128 bytes; stage into LDS
    const int ch = t & 7, lr0 = t >> 3;
    const int64_t gc = C0 + CH * ch;
    uint4 raw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t gr = R0 + lr0 + 32 * k;
        raw[k] = make_uint4(0u, 0u, 0u, 0u);
        if (gr < rows && gc < cols) raw[k] = *reinterpret_cast<const uint4*>(x + gr * ld + gc);
    }
    const TensorScale ts = prologue(amax_src, n_part, DO_ROW ? rts : nullptr, cts, amax_out);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int lr = lr0 + 32 * k;
        const int sw = (lr >> 4) & 15;
        uint8_t* rowp = tile + lr * STRIDE;
        *reinterpret_cast<uint2*>(rowp + 8 * ((2 * ch) ^ sw)) = make_uint2(raw[k].x, raw[k].y);
        *reinterpret_cast<uint2*>(rowp + 8 * ((2 * ch + 1) ^ sw)) = make_uint2(raw[k].z, raw[k].w);
    }
    if (DO_ROW) tile_row_blocks<T, SR>(raw, R0, lr0, gc, rows, cols, ts, seed, rcodes, rscales);
    __syncthreads();

    tile_col_blocks<T, SR, RHT>(tile, R0, C0, rows, cols, ts, seed, sign_mask, ccodes, cscales);
}

// ============================================================ BLK_2D
// A thread owns a 16-row x 8-column patch; lanes 2k and 2k+1 together hold one
// 16 x 16 square and combine their maxima with one lane exchange.  Wave w takes
// row band 4 * blockIdx.y + w; the 64 lanes cover 512 columns from
// 512 * blockIdx.x, so every 16-byte load of a wave reads 1 KiB of one
// row and every code store writes 256 contiguous bytes.
template <typename T, bool SR>
__global__ void __launch_bounds__(256) k_quant_2d(const T* __restrict__ x, int64_t rows,
                                                  int64_t cols, int64_t ld,
                                                  const float* __restrict__ amax_src, int n_part,
                                                  uint64_t seed, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ ts_out, float* amax_out) {
    const int lane = threadIdx.x & 63;
    const int64_t c = (int64_t)blockIdx.x * 512 + lane * 8;
    {
        const int64_t rband = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
        const int64_t r0 = rband * 16;
        const bool active = (r0 < rows) && (c < cols);
        // inactive lanes read a clamped in-range patch (never stored), so the
        // 16 loads carry no branch and issue together
        const int64_t rl = r0 < rows ? r0 : rows - 16, cl = c < cols ? c : cols - 8;
        float v[16][8];
#pragma unroll
        for (int i = 0; i < 16; ++i) load8(x + (rl + i) * ld + cl, v[i]);
        const TensorScale ts = prologue(amax_src, n_part, ts_out, nullptr, amax_out);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[i][e]));
        // the partner lane holds the other 8 columns of the square (both are
        // active or both inactive, since cols % 16 == 0)
        a = fmaxf(a, lane_xor1(a));
        if (!active) return;
        BlockScale bs = block_scale(a, ts.six_st, ts.rtab);
        if ((lane & 1) == 0) scales[rband * (cols / 16) + c / 16] = (uint8_t)bs.byte;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const int64_t r = r0 + i;
            uint32_t wd[2][4];
            if (SR) philox_words2(seed, kStream2D, (uint64_t)(r * cols + c), (uint64_t)((r + 1) * cols + c), wd[0], wd[1]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t w[1];
                encode<SR, 8, sizeof(T) == 2>(v[i + h], bs, a, wd[h], w);
                // non-temporal as in the row kernel (whole lines per wave)
                __builtin_nontemporal_store(w[0], reinterpret_cast<uint32_t*>(codes + (r + h) * (cols / 2) + c / 2));
            }
        }
    }
}

// ============================================================ dequantize
// A lane expands half of a 16-element block (8 elements: one code word and
// the block's multiplier) of each of 8 rows; the 64 lanes of a wave cover 32
// blocks (512 columns), so each wave-wide store writes 1 KiB (bf16; 2 KiB as
// two stores for fp32) of one row contiguously and each code load reads 256
// contiguous bytes.  WX of the four waves sit side by side (512 WX columns
// from 512 WX * blockIdx.x) on each of 4 / WX groups of 8 rows: with WX = 4 a
// 128-byte line of scale bytes (2048 columns) is read by one workgroup instead
// of four (against WX = 1, 8192^2 to BF16: 28.4 -> 26.7 us).  The launcher
// takes the largest WX whose span divides the width, so no wave idles at the
// right edge.  Codes are expanded two at a time by
// the gfx950 FP4 unpack instruction (scale operand 1.0, so the values are
// exact), then multiplied by the block multiplier (exact: at most 6
// significant bits) and by s_t (one rounding).
template <typename TOut, int WX>
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ ts, int64_t rows,
                                                 int64_t cols, int scale_2d, TOut* __restrict__ y,
                                                 int64_t ld) {
    const float st = ts[0];
    const int64_t nb = cols / 16;
    const int lane = threadIdx.x & 63;
    const int hf = lane & 1;
    const int wv = threadIdx.x >> 6;
    const int64_t b = (int64_t)blockIdx.x * (32 * WX) + 32 * (wv % WX) + (lane >> 1);
    if (b >= nb) return;
    constexpr int RG = 8 * (4 / WX);  // rows per workgroup
    const int64_t nrg = (rows + RG - 1) / RG;
    const int sshift = scale_2d ? 4 : 0;
    for (int64_t rg = blockIdx.y; rg < nrg; rg += gridDim.y) {
        const int64_t r0 = rg * RG + 8 * (wv / WX);
        uint32_t cw[8], sb[8];
        // rows past the end read the last row (never stored), and the scale
        // row is r >> 4 for 16x16 blocks, so the loads carry no branch and
        // issue back to back
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + i < rows ? r0 + i : rows - 1;
            cw[i] = *reinterpret_cast<const uint32_t*>(codes + (r * nb + b) * 8 + 4 * hf);
            sb[i] = scales[(r >> sshift) * nb + b];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + i;
            const float sv = e4m3_value(sb[i]);
            float o[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float2 p = e2m1x2_unpack(cw[i], k);
                o[2 * k] = (p.x * sv) * st;
                o[2 * k + 1] = (p.y * sv) * st;
            }
            if (r >= rows) continue;  // (only the stores are predicated)
            TOut* qp = y + r * ld + b * 16 + 8 * hf;
            if constexpr (sizeof(TOut) == 2) {
                // non-temporal: each wave store writes 1 KiB of one row, the
                // output is large and not read again here (8192^2: 35.3 ->
                // 29.3 us); the FP32 form, whose two stores per lane each
                // cover every other 16 bytes, ran 1.7x slower that way
                typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
                const v4u_t v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                 pack_bf16x2(o[6], o[7])};
                __builtin_nontemporal_store(v, reinterpret_cast<v4u_t*>(qp));
            } else {
                float4* qq = reinterpret_cast<float4*>(qp);
                qq[0] = make_float4(o[0], o[1], o[2], o[3]);
                qq[1] = make_float4(o[4], o[5], o[6], o[7]);
            }
        }
    }
}

// ============================================================ re-quantize
// Re-quantization of a row-blocked NVFP4 tensor along columns (the backward
// pass's transposed operand formed from the stored forward tensor, "Thinking
// Machines ускорила обучение Inkling 2 Small 4-битными числами", iitak.ru,
// section "Как это работает"): the result equals COL_1D quantization of the
// binary32 dequantization x = fl(fl(v * e4m3(sb)) * s_t).  The input is read
// as codes and scale bytes only (0.5625 bytes per element).

// Dequantized values of 8 consecutive elements of one row (one code word, one
// multiplier), exactly as k_dequant forms them.
__device__ __forceinline__ void dequant8(uint32_t w, float sv, float st, float v[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float2 p = e2m1x2_unpack(w, k);
        v[2 * k] = (p.x * sv) * st;
        v[2 * k + 1] = (p.y * sv) * st;
    }
}

// Partial maxima of |x| (RHT: of the transform of x down columns) over the
// dequantized tensor.  A thread takes a 16-row band x 8-column group (16 code
// words and 16 multipliers), groups along a band first.
template <bool RHT>
__global__ void __launch_bounds__(256) k_amax_req(const uint8_t* __restrict__ icodes,
                                                  const uint8_t* __restrict__ iscales,
                                                  const float* __restrict__ its, int64_t rows,
                                                  int64_t cols, uint32_t sign_mask,
                                                  float* __restrict__ partial) {
    const float st = its[0];
    const int64_t ng = cols / 8, nunits = (rows / 16) * ng;
    float a = 0.0f;
    for (int64_t un = (int64_t)(blockIdx.y * gridDim.x + blockIdx.x) * 256 + threadIdx.x; un < nunits;
         un += (int64_t)gridDim.x * gridDim.y * 256) {
        const int64_t band = un / ng, g = un % ng;
        float v[16][8];
        uint32_t w[16], sb[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t r = band * 16 + i;
            w[i] = *reinterpret_cast<const uint32_t*>(icodes + r * (cols / 2) + g * 4);
            sb[i] = iscales[r * (cols / 16) + g / 2];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) dequant8(w[i], e4m3_value(sb[i]), st, v[i]);
        if (RHT) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float col[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) col[i] = v[i][e];
                a = fmaxf(a, hadamard16_absmax(col, sign_mask));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[i][e]));
        }
    }
    store_partial(a, partial);
}

// Workgroup (x, y) takes rows 256 y .. + 255 and kReqTiles = 8 consecutive
// tiles of 32 columns from 256 x: per row 128 bytes of codes (one whole cache
// line) and 16 scale bytes.
//   load: thread t reads 16-byte code chunk t % 8 of rows t / 8 + 32 k
//     (k = 0..7), so 8 lanes cover one row's line, and row t's 16 scale
//     bytes; the codes go to LDS raw, chunk c of row r at chunk c ^ (r % 8);
//   per tile: thread t takes row t's chunk of that tile (32 codes) and its two
//     multipliers, dequantizes them into binary32 in the LDS layout of the
//     FP32 column tile, and the column phase runs exactly as for FP32 input.
// A workgroup re-quantizes a tile of 256 rows x 256 columns.  Its codes (128
// bytes of each row, 16-byte chunk t % 8 of rows t / 8 + 32 k, so every wave
// load reads 8 whole 128-byte lines) go to LDS in the transpose tile's layout
// (8-byte unit j of row r at unit j ^ (r / 16 % 16), rows 136 bytes apart),
// and its scale bytes transposed (the bytes of column block u for rows
// 4m .. 4m + 3 in dword 65 u + m).  After the one barrier, thread t takes row
// band t % 16 and column block t / 16 (16 rows x 16 columns): 16 8-byte code
// reads and 4 scale-dword reads give it the block, which it dequantizes one
// column pair at a time (x = fl(fl(v * e4m3(sb)) * s_t), as dequant8) into the
// column encoder of the transpose tile.  The 16 lanes of a column block share
// it, so each wave-wide code store writes 4 whole 128-byte lines.  Workgroups
// are grouped by XCD in runs of 8 tiles along x (xcd_tile), so the 8
// workgroups that share each 128-byte line of scale bytes read it through one
// L2.  (Against 8 phases of 32 columns staged as binary32 through LDS, with
// 16 barriers and 68 KB of LDS per workgroup, on 8192^2: see the launcher.)
template <bool SR, bool RHT>
__global__ void __launch_bounds__(256) k_requant_col(const uint8_t* __restrict__ icodes,
                                                     const uint8_t* __restrict__ iscales,
                                                     const float* __restrict__ its, int64_t rows,
                                                     int64_t cols, const float* __restrict__ amax_src,
                                                     int n_part, uint64_t seed, uint32_t sign_mask,
                                                     uint8_t* __restrict__ ccodes,
                                                     uint8_t* __restrict__ cscales,
                                                     float* __restrict__ cts, float* amax_out,
                                                     int xcd_group) {
    constexpr int STRIDE = 136;
    __shared__ __attribute__((aligned(16))) uint8_t ctile[256 * STRIDE];
    __shared__ uint32_t stile[16 * 65];
    const int t = threadIdx.x;
    const TileXY tl = xcd_tile_pairs(xcd_group);
    const int64_t R0 = tl.y * 256, C0 = tl.x * 256;
    const int64_t cb = cols / 2, sb = cols / 16;  // code and scale bytes per row

    // ---- codes.  Rows past the end read a clamped in-range row (their bands
    // are never encoded); a chunk with only 16 valid columns (cols % 32 == 16)
    // fills its upper half with zeros, and chunks past the last column load
    // nothing (neither is ever encoded).
    const int ch = t & 7, lr0 = t >> 3;
    const int64_t cc = C0 + 32 * ch;
    uint4 q[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t gr = min(R0 + lr0 + 32 * k, rows - 1);
        const uint8_t* cp = icodes + gr * cb + cc / 2;
        q[k] = make_uint4(0u, 0u, 0u, 0u);
        if (cc + 32 <= cols) {
            q[k] = *reinterpret_cast<const uint4*>(cp);
        } else if (cc < cols) {
            const uint2 lo = *reinterpret_cast<const uint2*>(cp);
            q[k] = make_uint4(lo.x, lo.y, 0u, 0u);
        }
    }
    // ---- scale bytes of row t for the 16 column blocks (clamped like the codes)
    const int64_t srow = min(R0 + t, rows - 1);
    uint32_t sv4[4];
    if (sb % 16 == 0 && (reinterpret_cast<uintptr_t>(iscales) & 15) == 0 && C0 + 256 <= cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(iscales + srow * sb + C0 / 16);
        sv4[0] = v.x; sv4[1] = v.y; sv4[2] = v.z; sv4[3] = v.w;
    } else {
        uint32_t b[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int64_t sc = C0 / 16 + j;
            b[j] = sc < sb ? iscales[srow * sb + sc] : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sv4[j] = b[4 * j] | (b[4 * j + 1] << 8) | (b[4 * j + 2] << 16) | (b[4 * j + 3] << 24);
    }
    const float st_in = its[0];
    const TensorScale ts = prologue(amax_src, n_part, cts, nullptr, amax_out);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int lr = lr0 + 32 * k;
        const int sw = (lr >> 4) & 15;
        uint8_t* rowp = ctile + lr * STRIDE;
        *reinterpret_cast<uint2*>(rowp + 8 * ((2 * ch) ^ sw)) = make_uint2(q[k].x, q[k].y);
        *reinterpret_cast<uint2*>(rowp + 8 * ((2 * ch + 1) ^ sw)) = make_uint2(q[k].z, q[k].w);
    }
    {
        uint8_t* const sbytes = reinterpret_cast<uint8_t*>(stile);
#pragma unroll
        for (int u = 0; u < 16; ++u) sbytes[4 * (65 * u + (t >> 2)) + (t & 3)] = (uint8_t)(sv4[u >> 2] >> (8 * (u & 3)));
    }
    __syncthreads();

    // ---- column blocks: band rb, column block u (16 columns)
    const int rb = t & 15, u = t >> 4;
    const int64_t r0 = R0 + 16 * rb, c0 = C0 + 16 * u;
    if (r0 >= rows || c0 >= cols) return;  // (rows, cols % 16 == 0: whole blocks; no barrier follows)
    uint2 w16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w16[i] = *reinterpret_cast<const uint2*>(ctile + (16 * rb + i) * STRIDE + 8 * (u ^ rb));
    float sv[16];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t d = stile[65 * u + 4 * rb + m];
#pragma unroll
        for (int j = 0; j < 4; ++j) sv[4 * m + j] = e4m3_value((d >> (8 * j)) & 0xFFu);
    }
    uint32_t sflip[16];
    sign_flips16(sign_mask, sflip);
    // the lane's output addresses and draw index for column c0, stepped by
    // wave-uniform multiples of a column
    uint8_t* const cdst0 = ccodes + c0 * (rows / 2) + r0 / 2;
    uint8_t* const csdst0 = cscales + c0 * (rows / 16) + r0 / 16;
    const uint64_t cidx0 = (uint64_t)(c0 * rows + r0);
    // (a rolled loop over the column pairs; each row's code word is shifted a
    // byte per pair rather than indexed, which would put w16 in scratch)
    uint32_t wcur[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) wcur[i] = w16[i].x;
#pragma unroll 1
    for (int p = 0; p < 8; ++p) {
        // columns 2p and 2p + 1: code byte p of every row, now byte 0 of wcur
        uint2 x2[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float2 v = e2m1x2_unpack(wcur[i], 0);
            x2[i] = make_uint2(__float_as_uint((v.x * sv[i]) * st_in), __float_as_uint((v.y * sv[i]) * st_in));
            wcur[i] = p == 3 ? w16[i].y : wcur[i] >> 8;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int64_t j = 2 * p + e;
            uint32_t cw[2];
            const BlockScale bs =
                col_unit_block<float, SR, RHT>(x2, e, sflip, sign_mask, ts, seed, cidx0 + (uint64_t)j * rows, cw);
            // non-temporal as in the column kernels: the 16 lanes of a column
            // write one whole 128-byte line
            typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
            const v2u_t cv = {cw[0], cw[1]};
            __builtin_nontemporal_store(cv, reinterpret_cast<v2u_t*>(cdst0 + j * (rows / 2)));
            csdst0[j * (rows / 16)] = (uint8_t)bs.byte;
        }
    }
}

// ============================================================ host launchers
namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// grid y covers `units` row groups, capped (the kernels loop over the rest)
inline unsigned grid_y(int64_t units) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>(units, 65535)); }

// Launch the amax pass; returns the number of partials written to ws
// (at most kMaxPartials).
template <typename T>
int amax_partials(const T* x, int64_t rows, int64_t cols, int64_t ld, int hadamard_dim,
                  uint32_t sign_mask, float* ws, hipStream_t s) {
    constexpr int CH = 16 / sizeof(T);
    int64_t gx, gy;
    if (hadamard_dim == 1) {          // along rows
        gx = std::min<int64_t>(std::max<int64_t>(cdiv(cols / 16, 512), 1), kMaxPartials);
        gy = std::min<int64_t>(std::max<int64_t>(rows, 1), kMaxPartials / gx);
        hipLaunchKernelGGL(k_amax_hadamard_rows<T>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x,
                           rows, cols, ld, sign_mask, ws);
    } else if (hadamard_dim == 2) {   // down columns
        // a workgroup takes whole 16-row bands (contiguous in memory) when
        // there are enough of them to fill the partials; split across
        // columns only when there are not (8192 x 20480 BF16 with the
        // amax computed: 172 -> 168 us against bands cut in 5)
        const int64_t nb = std::max<int64_t>(rows / 16, 1);
        gx = std::min<int64_t>(std::max<int64_t>(cdiv(cdiv(cols, CH), kAmaxColsThreads), 1),
                               std::max<int64_t>(kMaxPartials / nb, 1));
        gy = std::min<int64_t>(nb, kMaxPartials / gx);
        hipLaunchKernelGGL(k_amax_hadamard_cols<T>, dim3((unsigned)gx, (unsigned)gy), dim3(kAmaxColsThreads), 0, s, x,
                           rows, cols, ld, sign_mask, ws);
    } else {
        // a contiguous tensor streams as one long row
        const bool flat = (ld == cols) || rows == 1;
        const int64_t r = flat ? 1 : rows, c = flat ? rows * cols : cols;
        gx = std::min<int64_t>(std::max<int64_t>(cdiv(cdiv(c, CH), 2048), 1), kMaxPartials);
        gy = std::min<int64_t>(r, kMaxPartials / gx);
        hipLaunchKernelGGL(k_amax_plain<T>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, x, r, c,
                           flat ? c : ld, ws);
    }
    return (int)(gx * gy);
}

template <typename T>
hipError_t quantize_typed(const T* x, int64_t rows, int64_t cols, int64_t ld, int layout, bool sr,
                          uint64_t seed, bool rht, uint64_t hseed, const float* amax_in,
                          float* amax_out, const QOut* out, float* ws, hipStream_t s) {
    if (layout == kLayoutRowCol && rht) {
        // The two outputs quantize two different tensors: x transformed along
        // rows (row blocks) and x transformed down columns (column blocks),
        // each with its own A_t; amax_in / amax_out hold those two values, the
        // row output's first.  The two calls run in stream order, so the
        // second amax pass reuses the workspace after the first call is done
        // with it.
        hipError_t e = quantize_typed(x, rows, cols, ld, kLayoutRow, sr, seed, true, hseed, amax_in,
                                      amax_out, &out[0], ws, s);
        if (e != hipSuccess) return e;
        return quantize_typed(x, rows, cols, ld, kLayoutCol, sr, seed, true, hseed,
                              amax_in ? amax_in + 1 : nullptr, amax_out ? amax_out + 1 : nullptr,
                              &out[1], ws, s);
    }
    const uint32_t mask = rht ? hadamard_sign_mask(hseed) : 0u;
    if (rows == 0 || cols == 0) {
        hipLaunchKernelGGL(k_write_tensor_scale, dim3(1), dim3(1), 0, s, amax_in, out[0].ts,
                           layout == kLayoutRowCol ? out[1].ts : nullptr, amax_out);
        return hipGetLastError();
    }
    const float* amax = amax_in;
    int np = 0;
    if (!amax) {
        const int hdim = rht ? ((layout == kLayoutCol) ? 2 : 1) : 0;
        np = amax_partials(x, rows, cols, ld, hdim, mask, ws, s);
        amax = ws;
    }
    const QOut& o = out[0];
    switch (layout) {
        case kLayoutRow: {
            dim3 g((unsigned)cdiv(cols, 512), grid_y(cdiv(rows, 8)));
#define NVFP4_ROW(SRV, RHTV)                                                                         \
    hipLaunchKernelGGL((k_quant_row<T, SRV, RHTV>), g, dim3(256), 0, s, x, rows, cols, ld, amax, np, \
                       seed, mask, o.codes, o.scales, o.ts, amax_out)
            if (sr) {
                if (rht) NVFP4_ROW(true, true); else NVFP4_ROW(true, false);
            } else {
                if (rht) NVFP4_ROW(false, true); else NVFP4_ROW(false, false);
            }
#undef NVFP4_ROW
            break;
        }
        case kLayoutCol:
        case kLayoutRowCol: {
            dim3 g((unsigned)cdiv(cols, ColTile<T>::TWC), (unsigned)cdiv(rows, 256));
            // runs of tiles along a tile row share one XCD.  Fused layout: a
            // 128-byte line of row codes spans 4 (bf16) or 8 (fp32) tiles, a
            // line of row scales 32 or 64.  Column layout with nearest-even
            // rounding: an XCD then reads xg * 128 contiguous bytes of each
            // row (8192^2 bf16: 36.7 -> 34.3 us); with stochastic rounding
            // the same grouping measured 6% slower, so it keeps the
            // dispatch order
            const bool group = layout == kLayoutRowCol || !sr;
            const int xg = !group ? 1
                           : (g.x % (16 * sizeof(T)) == 0) ? (int)(16 * sizeof(T))
                           : (g.x % (2 * sizeof(T)) == 0) ? (int)(2 * sizeof(T)) : 1;
            const QOut& r = out[0];
            const QOut& c = layout == kLayoutCol ? out[0] : out[1];
#define NVFP4_TILE(ROWV, SRV, RHTV)                                                                  \
    hipLaunchKernelGGL((k_quant_colt<T, ROWV, SRV, RHTV>), g, dim3(256), 0, s, x, rows, cols, ld,   \
                       amax, np, seed, mask, r.codes, r.scales, r.ts, c.codes, c.scales, c.ts,      \
                       amax_out, xg)
            if (layout == kLayoutCol) {
                if (sr) {
                    if (rht) NVFP4_TILE(false, true, true); else NVFP4_TILE(false, true, false);
                } else {
                    if (rht) NVFP4_TILE(false, false, true); else NVFP4_TILE(false, false, false);
                }
            } else {
                if (sr) NVFP4_TILE(true, true, false); else NVFP4_TILE(true, false, false);
            }
#undef NVFP4_TILE
            break;
        }
        case kLayout2D: {
            dim3 g((unsigned)cdiv(cols, 512), (unsigned)cdiv(rows / 16, 4));
            if (sr)
                hipLaunchKernelGGL((k_quant_2d<T, true>), g, dim3(256), 0, s, x, rows, cols, ld, amax,
                                   np, seed, o.codes, o.scales, o.ts, amax_out);
            else
                hipLaunchKernelGGL((k_quant_2d<T, false>), g, dim3(256), 0, s, x, rows, cols, ld, amax,
                                   np, seed, o.codes, o.scales, o.ts, amax_out);
            break;
        }
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           int layout, bool sr, uint64_t seed, bool rht, uint64_t hseed,
                           const float* amax_in, float* amax_out, const QOut* out, float* ws,
                           hipStream_t s) {
    if (bf16)
        return quantize_typed(static_cast<const uint16_t*>(x), rows, cols, ld, layout, sr, seed, rht,
                              hseed, amax_in, amax_out, out, ws, s);
    return quantize_typed(static_cast<const float*>(x), rows, cols, ld, layout, sr, seed, rht, hseed,
                          amax_in, amax_out, out, ws, s);
}

hipError_t launch_requantize(const uint8_t* icodes, const uint8_t* iscales, const float* its,
                             int64_t rows, int64_t cols, bool sr, uint64_t seed, bool rht,
                             uint64_t hseed, const float* amax_in, float* amax_out, const QOut* out,
                             float* ws, hipStream_t s) {
    const uint32_t mask = rht ? hadamard_sign_mask(hseed) : 0u;
    if (rows == 0 || cols == 0) {
        hipLaunchKernelGGL(k_write_tensor_scale, dim3(1), dim3(1), 0, s, amax_in, out->ts, nullptr,
                           amax_out);
        return hipGetLastError();
    }
    const float* amax = amax_in;
    int np = 0;
    if (!amax) {
        const int64_t units = (rows / 16) * (cols / 8);
        const unsigned gx = (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(units, 256 * 4), kMaxPartials));
        if (rht)
            hipLaunchKernelGGL(k_amax_req<true>, dim3(gx), dim3(256), 0, s, icodes, iscales, its, rows,
                               cols, mask, ws);
        else
            hipLaunchKernelGGL(k_amax_req<false>, dim3(gx), dim3(256), 0, s, icodes, iscales, its, rows,
                               cols, mask, ws);
        amax = ws;
        np = (int)gx;
    }
    // (8192^2, stochastic rounding: 50.5 us with 8 binary32 phases per
    // workgroup, see the kernel)
    dim3 g((unsigned)cdiv(cols, 256), (unsigned)cdiv(rows, 256));
    // runs of 8 tiles along x share their scale-byte lines: one XCD each
    const int xg = g.x % 8 == 0 ? 8 : 1;
#define NVFP4_REQ(SRV, RHTV)                                                                       \
    hipLaunchKernelGGL((k_requant_col<SRV, RHTV>), g, dim3(256), 0, s, icodes, iscales, its, rows, \
                       cols, amax, np, seed, mask, out->codes, out->scales, out->ts, amax_out, xg)
    if (sr) {
        if (rht) NVFP4_REQ(true, true); else NVFP4_REQ(true, false);
    } else {
        if (rht) NVFP4_REQ(false, true); else NVFP4_REQ(false, false);
    }
#undef NVFP4_REQ
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts,
                             int64_t rows, int64_t cols, bool scale_2d, void* y, bool bf16,
                             int64_t ld, hipStream_t s) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int wx = cols % 2048 == 0 ? 4 : cols % 1024 == 0 ? 2 : 1;
    dim3 g((unsigned)cdiv(cols / 16, 32 * wx), grid_y(cdiv(rows, 8 * (4 / wx))));
#define NVFP4_DQ(TO, WXV)                                                                    \
    hipLaunchKernelGGL((k_dequant<TO, WXV>), g, dim3(256), 0, s, codes, scales, ts, rows, cols, \
                       (int)scale_2d, static_cast<TO*>(y), ld)
    if (bf16) {
        if (wx == 4) NVFP4_DQ(uint16_t, 4); else if (wx == 2) NVFP4_DQ(uint16_t, 2); else NVFP4_DQ(uint16_t, 1);
    } else {
        if (wx == 4) NVFP4_DQ(float, 4); else if (wx == 2) NVFP4_DQ(float, 2); else NVFP4_DQ(float, 1);
    }
#undef NVFP4_DQ
    return hipGetLastError();
}

}  // namespace nvfp4
