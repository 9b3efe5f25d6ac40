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
// All of these are HBM-bound streaming kernels.  Shared structure:
//   - 256-thread workgroups (four wave64s), 16-byte vector loads whose lanes
//     cover contiguous addresses, and stores that are contiguous across lanes;
//   - the tensor amax is a separate pass (per-workgroup partial maxima, then one
//     small reduction) unless the caller supplies it, because the block
//     multiplier of every block depends on it;
//   - the column layout stages a 64 x 64 tile in LDS so that both the loads
//     (along input rows) and the stores (along output rows, i.e. input columns)
//     stay contiguous.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

// ============================================================ amax
// Per-workgroup partial maxima of |x| over a rows x cols tensor (no transform),
// visiting 16-byte chunks along rows.  partial[blockIdx] is always written.
template <typename T>
__global__ void __launch_bounds__(256) k_amax_plain(const T* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld,
                                                    float* __restrict__ partial) {
    constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
    const int64_t nch = (cols + CH - 1) / CH;
    float a = 0.0f;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const T* row = x + r * ld;
        for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nch; j += (int64_t)gridDim.x * 256) {
            float v[8];
            if constexpr (sizeof(T) == 2) {
                load8(reinterpret_cast<const uint16_t*>(row) + j * CH, v);
            } else {
                float4 q = *reinterpret_cast<const float4*>(row + j * CH);
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            }
            int64_t valid = cols - j * CH;
#pragma unroll
            for (int e = 0; e < CH; ++e)
                if (e < valid) a = fmaxf(a, fabsf(v[e]));
        }
    }
    // wave reduction then workgroup reduction
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0)
        partial[blockIdx.y * gridDim.x + blockIdx.x] =
            fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Partial maxima of |H16 D x| with the transform applied along rows (groups
// of 16 consecutive columns; cols % 16 == 0).
template <typename T>
__global__ void __launch_bounds__(256) k_amax_hadamard_rows(const T* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ld,
                                                            uint32_t sign_mask,
                                                            float* __restrict__ partial) {
    const int64_t nb = cols / 16;
    float a = 0.0f;
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
        const T* row = x + r * ld;
        for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nb; j += (int64_t)gridDim.x * 256) {
            float v[16];
            load8(row + j * 16, v);
            load8(row + j * 16 + 8, v + 8);
            hadamard16(v, sign_mask);
            a = fmaxf(a, absmax16(v));
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0)
        partial[blockIdx.y * gridDim.x + blockIdx.x] =
            fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Partial maxima with the transform applied down columns (groups of 16
// consecutive rows; rows % 16 == 0).  A thread owns a 16-row x 16-byte patch.
template <typename T>
__global__ void __launch_bounds__(256) k_amax_hadamard_cols(const T* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ld,
                                                            uint32_t sign_mask,
                                                            float* __restrict__ partial) {
    constexpr int CH = 16 / sizeof(T);
    const int64_t nch = (cols + CH - 1) / CH;
    const int64_t nrb = rows / 16;
    float a = 0.0f;
    for (int64_t rb = blockIdx.y; rb < nrb; rb += gridDim.y) {
        for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nch; j += (int64_t)gridDim.x * 256) {
            float col[CH][16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const T* p = x + (rb * 16 + i) * ld + j * CH;
                float v[8];
                if constexpr (sizeof(T) == 2) {
                    load8(reinterpret_cast<const uint16_t*>(p), v);
                } else {
                    float4 q = *reinterpret_cast<const float4*>(p);
                    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
                }
#pragma unroll
                for (int e = 0; e < CH; ++e) col[e][i] = v[e];
            }
            int64_t valid = cols - j * CH;
#pragma unroll
            for (int e = 0; e < CH; ++e) {
                hadamard16(col[e], sign_mask);
                if (e < valid) a = fmaxf(a, absmax16(col[e]));
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0)
        partial[blockIdx.y * gridDim.x + blockIdx.x] =
            fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One workgroup: out[0] = max(partial[0 .. n)).
__global__ void __launch_bounds__(256) k_amax_final(const float* __restrict__ partial, int n,
                                                    float* __restrict__ out) {
    float a = 0.0f;
    for (int i = threadIdx.x; i < n; i += 256) a = fmaxf(a, partial[i]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) out[0] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// tensor_scale outputs of an empty tensor (no element kernel runs).
__global__ void k_write_tensor_scale(const float* amax_in, float* ts0, float* ts1) {
    float st = tensor_scale_of(amax_in ? amax_in[0] : 0.0f);
    if (ts0) ts0[0] = st;
    if (ts1) ts1[0] = st;
}

// ============================================================ ROW_1D
// Workgroup = 4 waves x 4 rows (rows 16*blockIdx.x ..); lane l of a wave owns
// block (blockIdx.y * 64 + l) of each of its rows: 32 bytes of bf16 (or 64 of
// fp32) in, 8 code bytes and one scale byte out.  The lanes of a wave cover
// 2 (4) KiB of one row.
template <typename T, bool SR, bool RHT>
__global__ void __launch_bounds__(256) k_quant_row(const T* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld,
                                                   const float* __restrict__ amax_ptr,
                                                   uint64_t seed, uint32_t sign_mask,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales,
                                                   float* __restrict__ ts_out) {
    const float st = tensor_scale_of(amax_ptr[0]);
    const float six_st = 6.0f * st;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) ts_out[0] = st;
    const int64_t nb = cols / 16;
    const int64_t b = (int64_t)blockIdx.y * 64 + (threadIdx.x & 63);
    if (b >= nb) return;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + i;
        if (r >= rows) break;
        const T* p = x + r * ld + b * 16;
        float v[16];
        load8(p, v);
        load8(p + 8, v + 8);
        if (RHT) hadamard16(v, sign_mask);
        BlockScale bs = block_scale(absmax16(v), six_st, st);
        uint32_t d[16];
        if (SR) draws16(seed, kStreamRow, (uint64_t)(r * cols + b * 16), d);
        uint32_t w[2];
        encode<SR, 16>(v, bs, d, w);
        const int64_t blk = r * nb + b;
        *reinterpret_cast<uint2*>(codes + blk * 8) = make_uint2(w[0], w[1]);
        scales[blk] = (uint8_t)bs.byte;
    }
}

// ============================================================ tiles through LDS
// A 64 x 64 tile of x (rows r0.., cols c0..) as binary32 in LDS, row stride 65
// floats (the odd stride spreads column walks over the banks).
constexpr int kTile = 64;
constexpr int kTileStride = 65;

template <typename T>
__device__ __forceinline__ void load_tile(const T* __restrict__ x, int64_t rows, int64_t cols,
                                          int64_t ld, int64_t r0, int64_t c0, float* tile) {
    constexpr int CH = 16 / sizeof(T);           // elements per 16-byte chunk
    constexpr int NCH = kTile / CH;              // chunks per tile row
    constexpr int PER = kTile * NCH / 256;       // chunks per thread
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int idx = threadIdx.x + 256 * k;
        const int tr = idx / NCH, tc = (idx % NCH) * CH;
        const int64_t r = r0 + tr, c = c0 + tc;
        float v[8];
        if (r < rows && c < cols) {
            const T* p = x + r * ld + c;
            if constexpr (sizeof(T) == 2) {
                load8(reinterpret_cast<const uint16_t*>(p), v);
            } else {
                float4 q = *reinterpret_cast<const float4*>(p);
                v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < CH; ++e) v[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < CH; ++e) tile[tr * kTileStride + tc + e] = v[e];
    }
}

// Column blocks of the tile: thread t quantizes column c0 + t/4, rows
// r0 + 16*(t%4) .. +15, into row (c0 + t/4) of the transposed output.
template <bool SR, bool RHT>
__device__ __forceinline__ void quant_tile_cols(const float* tile, int64_t rows, int64_t cols,
                                                int64_t r0, int64_t c0, float st, float six_st,
                                                uint64_t seed, uint32_t sign_mask,
                                                uint8_t* __restrict__ codes,
                                                uint8_t* __restrict__ scales) {
    const int tc = threadIdx.x >> 2, rb = threadIdx.x & 3;
    const int64_t c = c0 + tc, r = r0 + 16 * rb;
    if (c >= cols || r >= rows) return;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = tile[(16 * rb + i) * kTileStride + tc];
    if (RHT) hadamard16(v, sign_mask);
    BlockScale bs = block_scale(absmax16(v), six_st, st);
    uint32_t d[16];
    if (SR) draws16(seed, kStreamCol, (uint64_t)(c * rows + r), d);
    uint32_t w[2];
    encode<SR, 16>(v, bs, d, w);
    *reinterpret_cast<uint2*>(codes + c * (rows / 2) + r / 2) = make_uint2(w[0], w[1]);
    scales[c * (rows / 16) + r / 16] = (uint8_t)bs.byte;
}

// Row blocks of the tile: thread t quantizes row r0 + t/4, columns
// c0 + 16*(t%4) .. +15.
template <bool SR>
__device__ __forceinline__ void quant_tile_rows(const float* tile, int64_t rows, int64_t cols,
                                                int64_t r0, int64_t c0, float st, float six_st,
                                                uint64_t seed, uint8_t* __restrict__ codes,
                                                uint8_t* __restrict__ scales) {
    const int tr = threadIdx.x >> 2, cb = threadIdx.x & 3;
    const int64_t r = r0 + tr, c = c0 + 16 * cb;
    if (r >= rows || c >= cols) return;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = tile[tr * kTileStride + 16 * cb + i];
    BlockScale bs = block_scale(absmax16(v), six_st, st);
    uint32_t d[16];
    if (SR) draws16(seed, kStreamRow, (uint64_t)(r * cols + c), d);
    uint32_t w[2];
    encode<SR, 16>(v, bs, d, w);
    *reinterpret_cast<uint2*>(codes + r * (cols / 2) + c / 2) = make_uint2(w[0], w[1]);
    scales[r * (cols / 16) + c / 16] = (uint8_t)bs.byte;
}

// COL_1D: grid (rows/64 tiles, cols/64 tiles); consecutive workgroups walk down
// the rows so that their output segments of one transposed row are adjacent.
template <typename T, bool SR, bool RHT>
__global__ void __launch_bounds__(256) k_quant_col(const T* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld,
                                                   const float* __restrict__ amax_ptr,
                                                   uint64_t seed, uint32_t sign_mask,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales,
                                                   float* __restrict__ ts_out) {
    __shared__ float tile[kTile * kTileStride];
    const float st = tensor_scale_of(amax_ptr[0]);
    const float six_st = 6.0f * st;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) ts_out[0] = st;
    const int64_t r0 = (int64_t)blockIdx.x * kTile, c0 = (int64_t)blockIdx.y * kTile;
    load_tile(x, rows, cols, ld, r0, c0, tile);
    __syncthreads();
    quant_tile_cols<SR, RHT>(tile, rows, cols, r0, c0, st, six_st, seed, sign_mask, codes, scales);
}

// ROW_COL_1D: one read of each tile, both outputs.
template <typename T, bool SR>
__global__ void __launch_bounds__(256) k_quant_rowcol(const T* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ld,
                                                      const float* __restrict__ amax_ptr,
                                                      uint64_t seed, uint8_t* __restrict__ rcodes,
                                                      uint8_t* __restrict__ rscales,
                                                      float* __restrict__ rts,
                                                      uint8_t* __restrict__ ccodes,
                                                      uint8_t* __restrict__ cscales,
                                                      float* __restrict__ cts) {
    __shared__ float tile[kTile * kTileStride];
    const float st = tensor_scale_of(amax_ptr[0]);
    const float six_st = 6.0f * st;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        rts[0] = st;
        cts[0] = st;
    }
    const int64_t r0 = (int64_t)blockIdx.x * kTile, c0 = (int64_t)blockIdx.y * kTile;
    load_tile(x, rows, cols, ld, r0, c0, tile);
    __syncthreads();
    quant_tile_rows<SR>(tile, rows, cols, r0, c0, st, six_st, seed, rcodes, rscales);
    quant_tile_cols<SR, false>(tile, rows, cols, r0, c0, st, six_st, seed, 0u, ccodes, cscales);
}

// ============================================================ BLK_2D
// A thread owns a 16-row x 8-column patch; lanes 2k and 2k+1 together hold one
// 16 x 16 square and combine their maxima with one lane exchange.  Wave w of
// the workgroup takes row band 4*blockIdx.x + w; the 64 lanes cover 512
// columns (from 512*blockIdx.y), so every 16-byte load of a wave reads 1 KiB
// of one row.
template <typename T, bool SR>
__global__ void __launch_bounds__(256) k_quant_2d(const T* __restrict__ x, int64_t rows,
                                                  int64_t cols, int64_t ld,
                                                  const float* __restrict__ amax_ptr,
                                                  uint64_t seed, uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ ts_out) {
    const float st = tensor_scale_of(amax_ptr[0]);
    const float six_st = 6.0f * st;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) ts_out[0] = st;
    const int lane = threadIdx.x & 63;
    const int64_t rband = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t c = (int64_t)blockIdx.y * 512 + lane * 8;
    const int64_t r0 = rband * 16;
    const bool active = (r0 < rows) && (c < cols);
    float v[16][8];
    float a = 0.0f;
    if (active) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            load8(x + (r0 + i) * ld + c, v[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(v[i][e]));
        }
    }
    // partner lane holds the other 8 columns of the square (both are active or
    // both inactive, since cols % 16 == 0)
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    if (!active) return;
    BlockScale bs = block_scale(a, six_st, st);
    const int64_t ncb = cols / 16;
    if ((lane & 1) == 0) scales[rband * ncb + c / 16] = (uint8_t)bs.byte;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t r = r0 + i;
        uint32_t d[8];
        if (SR) draws8(seed, kStream2D, (uint64_t)(r * cols + c), d);
        uint32_t w[1];
        encode<SR, 8>(v[i], bs, d, w);
        *reinterpret_cast<uint32_t*>(codes + r * (cols / 2) + c / 2) = w[0];
    }
}

// ============================================================ dequantize
// Same geometry as the row quantizer (rows on grid x, 64-block column groups on
// grid y): a lane expands one 16-element block of each of 4 rows; 8 code bytes and a scale byte in, 32 (bf16) or 64 (fp32)
// bytes out.
template <typename TOut>
__global__ void __launch_bounds__(256) k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ ts, int64_t rows,
                                                 int64_t cols, int scale_2d, TOut* __restrict__ y,
                                                 int64_t ld) {
    const float st = ts[0];
    const int64_t nb = cols / 16;
    const int64_t b = (int64_t)blockIdx.y * 64 + (threadIdx.x & 63);
    if (b >= nb) return;
    const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + i;
        if (r >= rows) break;
        const uint2 cw = *reinterpret_cast<const uint2*>(codes + (r * nb + b) * 8);
        const uint32_t sb = scale_2d ? scales[(r / 16) * nb + b] : scales[r * nb + b];
        const float sv = e4m3_value(sb);
        float o[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            uint32_t code = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 15u;
            float p = e2m1_value(code) * sv;  // exact: at most 6 significant bits
            o[j] = p * st;
        }
        TOut* q = y + r * ld + b * 16;
        if constexpr (sizeof(TOut) == 2) {
            uint32_t pk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                uint32_t lo = __float_as_uint(o[2 * j]), hi = __float_as_uint(o[2 * j + 1]);
                lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;   // nearest-even to bf16
                hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
                pk[j] = lo | (hi << 16);
            }
            uint4* qq = reinterpret_cast<uint4*>(q);
            qq[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
            qq[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
        } else {
            float4* qq = reinterpret_cast<float4*>(q);
#pragma unroll
            for (int j = 0; j < 4; ++j) qq[j] = make_float4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
        }
    }
}

// ============================================================ host launchers
namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// grid of an amax pass: x covers `units_x` per-thread units (256 per
// workgroup), y covers `units_y` rows (or row bands); at most kMaxPartials
// workgroups in total, both loops grid-stride.
dim3 amax_grid(int64_t units_x, int64_t units_y) {
    int64_t gx = std::min<int64_t>(std::max<int64_t>(cdiv(units_x, 256), 1), kMaxPartials);
    int64_t gy = std::min<int64_t>(std::max<int64_t>(units_y, 1), kMaxPartials / gx);
    return dim3((unsigned)gx, (unsigned)gy, 1);
}

template <typename T>
hipError_t amax_typed(const T* x, int64_t rows, int64_t cols, int64_t ld, int hadamard_dim,
                      uint32_t sign_mask, float* ws, hipStream_t s) {
    float* out = ws;
    float* partial = ws + 4;
    dim3 g;
    if (hadamard_dim == 1) {          // along rows
        g = amax_grid(cols / 16, rows);
        hipLaunchKernelGGL(k_amax_hadamard_rows<T>, g, dim3(256), 0, s, x, rows, cols, ld, sign_mask, partial);
    } else if (hadamard_dim == 2) {   // down columns
        constexpr int CH = 16 / sizeof(T);
        g = amax_grid(cdiv(cols, CH), rows / 16);
        hipLaunchKernelGGL(k_amax_hadamard_cols<T>, g, dim3(256), 0, s, x, rows, cols, ld, sign_mask, partial);
    } else {
        constexpr int CH = 16 / sizeof(T);
        g = amax_grid(cdiv(cols, CH), rows);
        hipLaunchKernelGGL(k_amax_plain<T>, g, dim3(256), 0, s, x, rows, cols, ld, partial);
    }
    hipLaunchKernelGGL(k_amax_final, dim3(1), dim3(256), 0, s, partial, (int)(g.x * g.y), out);
    return hipGetLastError();
}

template <typename T, bool SR>
void launch_row(const T* x, int64_t rows, int64_t cols, int64_t ld, const float* amax, uint64_t seed,
                bool rht, uint32_t mask, const QOut& o, hipStream_t s) {
    dim3 g((unsigned)cdiv(rows, 16), (unsigned)cdiv(cols / 16, 64));
    if (rht)
        hipLaunchKernelGGL((k_quant_row<T, SR, true>), g, dim3(256), 0, s, x, rows, cols, ld, amax,
                           seed, mask, o.codes, o.scales, o.ts);
    else
        hipLaunchKernelGGL((k_quant_row<T, SR, false>), g, dim3(256), 0, s, x, rows, cols, ld, amax,
                           seed, mask, o.codes, o.scales, o.ts);
}

template <typename T, bool SR>
void launch_col(const T* x, int64_t rows, int64_t cols, int64_t ld, const float* amax, uint64_t seed,
                bool rht, uint32_t mask, const QOut& o, hipStream_t s) {
    dim3 g((unsigned)cdiv(rows, kTile), (unsigned)cdiv(cols, kTile));
    if (rht)
        hipLaunchKernelGGL((k_quant_col<T, SR, true>), g, dim3(256), 0, s, x, rows, cols, ld, amax,
                           seed, mask, o.codes, o.scales, o.ts);
    else
        hipLaunchKernelGGL((k_quant_col<T, SR, false>), g, dim3(256), 0, s, x, rows, cols, ld, amax,
                           seed, mask, o.codes, o.scales, o.ts);
}

template <typename T, bool SR>
void launch_rowcol(const T* x, int64_t rows, int64_t cols, int64_t ld, const float* amax,
                   uint64_t seed, const QOut& r, const QOut& c, hipStream_t s) {
    dim3 g((unsigned)cdiv(rows, kTile), (unsigned)cdiv(cols, kTile));
    hipLaunchKernelGGL((k_quant_rowcol<T, SR>), g, dim3(256), 0, s, x, rows, cols, ld, amax, seed,
                       r.codes, r.scales, r.ts, c.codes, c.scales, c.ts);
}

template <typename T, bool SR>
void launch_2d(const T* x, int64_t rows, int64_t cols, int64_t ld, const float* amax, uint64_t seed,
               const QOut& o, hipStream_t s) {
    dim3 g((unsigned)cdiv(rows / 16, 4), (unsigned)cdiv(cols, 512));
    hipLaunchKernelGGL((k_quant_2d<T, SR>), g, dim3(256), 0, s, x, rows, cols, ld, amax, seed,
                       o.codes, o.scales, o.ts);
}

template <typename T>
hipError_t quantize_typed(const T* x, int64_t rows, int64_t cols, int64_t ld, int layout, bool sr,
                          uint64_t seed, bool rht, uint64_t hseed, const float* amax_in,
                          const QOut* out, float* ws, hipStream_t s) {
    const uint32_t mask = rht ? hadamard_sign_mask(hseed) : 0u;
    if (rows == 0 || cols == 0) {
        hipLaunchKernelGGL(k_write_tensor_scale, dim3(1), dim3(1), 0, s, amax_in, out[0].ts,
                           layout == kLayoutRowCol ? out[1].ts : nullptr);
        return hipGetLastError();
    }
    const float* amax = amax_in;
    if (!amax) {
        int hdim = 0;
        if (rht) hdim = (layout == kLayoutCol) ? 2 : 1;
        hipError_t e = amax_typed(x, rows, cols, ld, hdim, mask, ws, s);
        if (e != hipSuccess) return e;
        amax = ws;
    }
    switch (layout) {
        case kLayoutRow:
            sr ? launch_row<T, true>(x, rows, cols, ld, amax, seed, rht, mask, out[0], s)
               : launch_row<T, false>(x, rows, cols, ld, amax, seed, rht, mask, out[0], s);
            break;
        case kLayoutCol:
            sr ? launch_col<T, true>(x, rows, cols, ld, amax, seed, rht, mask, out[0], s)
               : launch_col<T, false>(x, rows, cols, ld, amax, seed, rht, mask, out[0], s);
            break;
        case kLayoutRowCol:
            sr ? launch_rowcol<T, true>(x, rows, cols, ld, amax, seed, out[0], out[1], s)
               : launch_rowcol<T, false>(x, rows, cols, ld, amax, seed, out[0], out[1], s);
            break;
        case kLayout2D:
            sr ? launch_2d<T, true>(x, rows, cols, ld, amax, seed, out[0], s)
               : launch_2d<T, false>(x, rows, cols, ld, amax, seed, out[0], s);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           int layout, bool sr, uint64_t seed, bool rht, uint64_t hseed,
                           const float* amax_in, const QOut* out, float* ws, hipStream_t s) {
    if (bf16)
        return quantize_typed(static_cast<const uint16_t*>(x), rows, cols, ld, layout, sr, seed, rht,
                              hseed, amax_in, out, ws, s);
    return quantize_typed(static_cast<const float*>(x), rows, cols, ld, layout, sr, seed, rht, hseed,
                          amax_in, out, ws, s);
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts,
                             int64_t rows, int64_t cols, bool scale_2d, void* y, bool bf16,
                             int64_t ld, hipStream_t s) {
    if (rows == 0 || cols == 0) return hipSuccess;
    dim3 g((unsigned)cdiv(rows, 16), (unsigned)cdiv(cols / 16, 64));
    if (bf16)
        hipLaunchKernelGGL(k_dequant<uint16_t>, g, dim3(256), 0, s, codes, scales, ts, rows, cols,
                           (int)scale_2d, static_cast<uint16_t*>(y), ld);
    else
        hipLaunchKernelGGL(k_dequant<float>, g, dim3(256), 0, s, codes, scales, ts, rows, cols,
                           (int)scale_2d, static_cast<float*>(y), ld);
    return hipGetLastError();
}

}  // namespace nvfp4
