// MX (OCP Microscaling) quantize and dequantize kernels for gfx950.
//
// The pages name the MX formats without defining them: MXFP8 carries the
// backward pass at Thinking Machines ("Thinking Machines ускорила обучение
// Inkling 2 Small 4-битными числами", iitak.ru, section "Как это работает"),
// MXFP4 is the Open Compute Project format NVFP4 is measured against
// ("Nvidia добивается успеха с 4-битным форматом NVFP4", asector.ru, section
// "Перспективы и дальнейшие направления исследований"), and expert outputs
// travel in an 8.25-bit format (iitak.ru page, section "Но") -- 8-bit
// elements plus one 8-bit scale per 32.  The reading implemented here is the OCP Microscaling definition:
//   - 32 consecutive elements along the block dimension share one E8M0 scale
//     X = 2^s, s = floor(log2 max|V|) - emax (emax 8 for E4M3 elements, 2 for
//     E2M1), clamped to [-127, 127], -127 for an all-zero block; the scale
//     byte is s + 127;
//   - y = fl(|V| * 2^-s) (exact unless it underflows), rounded onto the
//     element grid to nearest-even or stochastically (16-bit Philox draw,
//     round up iff draw < fraction * 2^16), saturating at 448 (E4M3) or 6
//     (E2M1); the sign is copied.
// SR draws use the NVFP4 Philox convention with streams 4 (row blocks) and 5
// (column blocks), indexed by the element's row-major position in the
// output.
//
// All kernels here are HBM-bound streams with the same shape as the NVFP4
// ones: the row kernel gives each lane 8 consecutive elements (a 32-element
// block spans 4 lanes, joined by two lane exchanges); the column kernel
// stages a 256-row x 128-byte tile in LDS and gives each lane 16 rows of UE
// columns, a lane pair holding the two halves of each 32-row block.  The
// scale needs no division: its exponent comes from the block maximum's
// exponent field, and 2^-s is built from bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

enum : uint32_t { kStreamMxRow = 4, kStreamMxCol = 5 };

inline int64_t mx_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline unsigned mx_grid_y(int64_t units) {
    return (unsigned)std::max<int64_t>(1, std::min<int64_t>(units, 65535));
}

template <int ELEM>
constexpr int mx_emax() {
    return ELEM == kMxE4M3 ? 8 : 2;
}

// Scale exponent of a block whose largest magnitude is amax (finite, >= 0):
// for a normal amax with exponent field E, floor(log2 amax) = E - 127 and
// s = E - 127 - emax never exceeds 127 - emax; a zero or subnormal amax
// (E = 0) lands below -127 and is clamped there, as is any amax below
// 2^(emax - 126).
template <int ELEM>
__device__ __forceinline__ int mx_scale_exp(float amax) {
    const int E = (int)(__float_as_uint(amax) >> 23);
    return max(E - 127 - mx_emax<ELEM>(), -127);
}

// 2^-s as binary32 (s in [-127, 127 - emax], so the biased exponent 127 - s is
// in [emax, 254]: always a normal number).
__device__ __forceinline__ float mx_inv_scale(int s) { return __uint_as_float((uint32_t)(127 - s) << 23); }

// E4M3 codes of 8 values (sign copied), nearest-even: y = v * 2^-s keeps the
// sign, is clamped to +-448 (the FP8 convert does not saturate on its own)
// and converted two at a time; two byte permutes assemble the words.
__device__ __forceinline__ void e4m3x8_rne(const float* v, float p2, uint32_t out[2]) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float* p = v + 4 * k;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = __builtin_amdgcn_fmed3f(p[j] * p2, -448.0f, 448.0f);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], 0, false);
        out[k] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);  // low halves of lo, then hi
    }
}

// E4M3 code of one value by stochastic rounding with the 16-bit draw carried
// by `seed` (sr_seed form): y = min(|v| * 2^-s, 448) is rounded up to the 2^-29
// grid, and the gfx950 SR FP8 convert with scale operand 2^29 then rounds up
// exactly when draw < fraction * 2^16 (checked against that integer rule over
// 3.6e8 value/draw pairs covering every E4M3 interval, the subnormal range,
// values below 2^-27, saturation and both signs).  The code lands in byte 0
// of the result; the other bytes are unspecified.
__device__ __forceinline__ uint32_t e4m3_sr1(float v, float p2, uint32_t seed) {
    const float y = fminf(fabsf(v) * p2, 448.0f);
    const float z = __builtin_ceilf(y * 0x1p29f);
    const float zs = __uint_as_float(__float_as_uint(z) | (__float_as_uint(v) & 0x80000000u));
    return (uint32_t)__builtin_amdgcn_cvt_scalef32_sr_fp8_f32(0, zs, seed, 0x1p29f, 0);
}

// E4M3 codes of 8 values by stochastic rounding; w holds the Philox words of
// the 8 elements (draws of elements 2j, 2j+1 in word j).
__device__ __forceinline__ void e4m3x8_sr(const float* v, float p2, const uint32_t* w, uint32_t out[2]) {
    const uint32_t lo2 = 0x0C0C0400u;  // byte 0 of src1, byte 0 of src0, zero, zero
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        uint32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = e4m3_sr1(v[4 * k + j], p2, sr_seed(w[2 * k + (j >> 1)], j & 1));
        out[k] = __builtin_amdgcn_perm(c[1], c[0], lo2) | (__builtin_amdgcn_perm(c[3], c[2], lo2) << 16);
    }
}

// Codes of N = 8 or 16 consecutive elements of one block: E4M3 -> N bytes in
// N/4 words; E2M1 -> N nibbles in N/8 words (even element in the low nibble).
template <int ELEM, bool SR, int N>
__device__ __forceinline__ void mx_encode(const float* v, float p2, float amax, const uint32_t* w,
                                          uint32_t* out) {
    if constexpr (ELEM == kMxE4M3) {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) {
            if (SR) e4m3x8_sr(v + 8 * k, p2, w + 4 * k, out + 2 * k);
            else e4m3x8_rne(v + 8 * k, p2, out + 2 * k);
        }
    } else {
        // the NVFP4 encoder with the block multiplier R = 2^-s; |v| * R < 8,
        // so it always takes its instruction path
        BlockScale bs;
        bs.byte = 0u;
        bs.R = p2;
        encode<SR, N>(v, bs, amax, w, out);
    }
}

// ============================================================ ROW_1D
// Lane l of wave w holds elements c = 512 * blockIdx.x + 8 l .. c + 7 of rows
// 8 * rg + 2 w and +1 (one 16-byte bf16 load, two fp32 loads per row); lanes
// 4k .. 4k+3 hold one 32-element block.  Row groups rg = blockIdx.y,
// + gridDim.y, ... (the next group's loads are issued before the current
// group's stores).
template <typename T, int ELEM, bool SR>
__global__ void __launch_bounds__(256) k_mx_row(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                int64_t ld, uint64_t seed, uint8_t* __restrict__ codes,
                                                uint8_t* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int q = lane & 3;
    const int64_t c = (int64_t)blockIdx.x * 512 + 8 * lane;
    const bool col_ok = c < cols;  // cols % 32 == 0: the 4 lanes of a block agree
    // lanes past the last column and rows past the last row read a clamped
    // in-range chunk whose results are never stored
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
    for (;;) {
        const int64_t r = rg * 8 + 2 * (threadIdx.x >> 6);
        float a[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[k][e]));
            m = fmaxf(m, lane_xor1(m));
            a[k] = fmaxf(m, lane_xor2(m));
        }
        if (col_ok) {
            uint32_t wd[2][4];
            if (SR)
                philox_words2(seed, kStreamMxRow, (uint64_t)(r * cols + c), (uint64_t)((r + 1) * cols + c),
                              wd[0], wd[1]);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int64_t rr = r + k;
                if (rr >= rows) break;
                const int s = mx_scale_exp<ELEM>(a[k]);
                uint32_t w[2];
                mx_encode<ELEM, SR, 8>(v[k], mx_inv_scale(s), a[k], wd[k], w);
                if constexpr (ELEM == kMxE4M3)
                    *reinterpret_cast<uint2*>(codes + rr * cols + c) = make_uint2(w[0], w[1]);
                else
                    *reinterpret_cast<uint32_t*>(codes + rr * (cols / 2) + c / 2) = w[0];
                if (q == k) scales[rr * (cols / 32) + c / 32] = (uint8_t)(s + 127);
            }
        }
        rg += gridDim.y;
        if (rg >= nrg) break;
        load_group(rg);
    }
}

// ============================================================ COL_1D
// Workgroup (x, y) owns the tile of 256 rows from 256 y and 128 bytes of each
// row (TWC = 64 bf16 or 32 fp32 columns) from column TWC x.
//   load: thread t reads 16-byte chunk t % 8 of tile rows t / 8 + 32 k
//     (k = 0..7); the chunk's two 8-byte units land in LDS at unit
//     (2 ch + h) ^ (band % 16) of the row (band = row / 16; rows padded to
//     136 bytes) so the column reads below spread over the banks;
//   columns: thread t takes 16-row band t % 16 and 8-byte unit t / 16, i.e.
//     16 rows x UE columns (UE = 4 bf16 or 2 fp32); lanes 2k and 2k+1 hold
//     the two 16-row halves of a 32-row block and join their maxima with one
//     exchange.  For each column a lane writes 16 E4M3 bytes or 8 E2M1 bytes,
//     so the 16 lanes sharing a unit write one contiguous stretch of every
//     transposed row.
template <typename T, int ELEM, bool SR>
__global__ void __launch_bounds__(256) k_mx_col(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                int64_t ld, uint64_t seed, uint8_t* __restrict__ codes,
                                                uint8_t* __restrict__ scales, int xcd_group) {
    constexpr int CH = 16 / (int)sizeof(T), TWC = 128 / (int)sizeof(T), UE = 8 / (int)sizeof(T);
    constexpr int STRIDE = 136;
    __shared__ __attribute__((aligned(16))) uint8_t tile[256 * STRIDE];
    const int t = threadIdx.x;
    const TileXY tl = xcd_tile(xcd_group);
    const int64_t R0 = tl.y * 256, C0 = tl.x * TWC;

    const int ch = t & 7, lr0 = t >> 3;
    const int64_t gc = C0 + CH * ch;
    // out-of-range rows and chunks read an in-range chunk that is never stored
    const int64_t gcl = gc < cols ? gc : 0;
    uint4 raw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t gr = R0 + lr0 + 32 * k;
        raw[k] = *reinterpret_cast<const uint4*>(x + (gr < rows ? gr : rows - 1) * ld + gcl);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int lr = lr0 + 32 * k;
        const int sw = (lr >> 4) & 15;
        uint8_t* rowp = tile + lr * STRIDE;
        *reinterpret_cast<uint2*>(rowp + 8 * ((2 * ch) ^ sw)) = make_uint2(raw[k].x, raw[k].y);
        *reinterpret_cast<uint2*>(rowp + 8 * ((2 * ch + 1) ^ sw)) = make_uint2(raw[k].z, raw[k].w);
    }
    __syncthreads();

    const int rb = t & 15, u = t >> 4;
    const int64_t r0 = R0 + 16 * rb;
    if (r0 >= rows) return;  // rows % 32 == 0: both halves of a block are in or out
    uint2 qv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        qv[i] = *reinterpret_cast<const uint2*>(tile + (16 * rb + i) * STRIDE + 8 * (u ^ rb));
#pragma unroll
    for (int e = 0; e < UE; ++e) {
        const int64_t c = C0 + UE * u + e;
        if (c >= cols) continue;  // the lane pair shares u, hence c
        float col[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if constexpr (sizeof(T) == 2) {
                const uint32_t wv = (e >> 1) == 0 ? qv[i].x : qv[i].y;
                col[i] = (e & 1) ? __uint_as_float(wv & 0xFFFF0000u) : __uint_as_float(wv << 16);
            } else {
                col[i] = __uint_as_float(e == 0 ? qv[i].x : qv[i].y);
            }
        }
        float a = absmax16(col);
        a = fmaxf(a, lane_xor1(a));
        const int s = mx_scale_exp<ELEM>(a);
        uint32_t wd[8];
        if (SR) philox_words16(seed, kStreamMxCol, (uint64_t)(c * rows + r0), wd);
        if constexpr (ELEM == kMxE4M3) {
            uint32_t w[4];
            mx_encode<ELEM, SR, 16>(col, mx_inv_scale(s), a, wd, w);
            *reinterpret_cast<uint4*>(codes + c * rows + r0) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            uint32_t w[2];
            mx_encode<ELEM, SR, 16>(col, mx_inv_scale(s), a, wd, w);
            *reinterpret_cast<uint2*>(codes + c * (rows / 2) + r0 / 2) = make_uint2(w[0], w[1]);
        }
        if ((rb & 1) == 0) scales[c * (rows / 32) + r0 / 32] = (uint8_t)(s + 127);
    }
}

// ============================================================ dequantize
// y = value(code) * 2^(byte - 127), one binary32 rounding (ldexp; exact
// unless the result leaves the normal range), BF16 output rounded to nearest
// even from that binary32 value.  A lane expands 8 elements (8 E4M3 code
// bytes or 4 E2M1 ones) of each of 8 rows; the 64 lanes of a wave cover 512
// elements of a row, so each wave-wide store writes 1 KiB (bf16) of a row
// contiguously.  WX of the four waves sit side by side on each of 4 / WX
// groups of 8 rows: with WX = 4 a 128-byte line of scale bytes (4096
// elements) is read by two workgroups instead of eight.  The launcher takes
// the largest WX whose span (512 WX elements) divides the width.  (With 16 elements per lane its two 16-byte stores each
// covered every other 16 bytes of 2 KiB: 8192^2 to BF16, alternating builds on
// one box, E2M1 44.2 -> 35.3 us, E4M3 42.4 -> 40.2 us.)
template <int ELEM, typename TOut, int WX>
__global__ void __launch_bounds__(256) k_mx_dequant(const uint8_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales, int64_t rows,
                                                    int64_t cols, TOut* __restrict__ y, int64_t ld) {
    constexpr int EPL = 8;                            // elements per lane
    constexpr int CB = ELEM == kMxE4M3 ? 8 : 4;       // their code bytes
    const int64_t row_bytes = ELEM == kMxE4M3 ? cols : cols / 2;
    const int wv = threadIdx.x >> 6;
    const int64_t b = (int64_t)blockIdx.x * (64 * WX) + 64 * (wv % WX) + (threadIdx.x & 63);
    if (b >= cols / EPL) return;
    constexpr int RG = 8 * (4 / WX);  // rows per workgroup
    const int64_t nrg = (rows + RG - 1) / RG;
    for (int64_t rg = blockIdx.y; rg < nrg; rg += gridDim.y) {
        const int64_t r0 = rg * RG + 8 * (wv / WX);
        uint32_t cw[8][2];
        int sx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + i < rows ? r0 + i : rows - 1;  // clamped; never stored
            if constexpr (CB == 8) {
                const uint2 q = *reinterpret_cast<const uint2*>(codes + r * row_bytes + CB * b);
                cw[i][0] = q.x; cw[i][1] = q.y;
            } else {
                cw[i][0] = *reinterpret_cast<const uint32_t*>(codes + r * row_bytes + CB * b);
                cw[i][1] = 0u;
            }
            sx[i] = (int)scales[r * (cols / 32) + (b * EPL) / 32] - 127;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + i;
            if (r >= rows) break;
            float o[EPL];
#pragma unroll
            for (int k = 0; k < EPL / 2; ++k) {
                float2 p;
                if constexpr (ELEM == kMxE4M3) {
                    if (k & 1) {
                        const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i][k >> 1], true);
                        p = make_float2(f[0], f[1]);
                    } else {
                        const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i][k >> 1], false);
                        p = make_float2(f[0], f[1]);
                    }
                } else {
                    p = e2m1x2_unpack(cw[i][0], k);
                }
                o[2 * k] = __builtin_amdgcn_ldexpf(p.x, sx[i]);
                o[2 * k + 1] = __builtin_amdgcn_ldexpf(p.y, sx[i]);
            }
            // non-temporal stores: the output is large and not read again here
            // (8192^2: E2M1 to BF16 35.4 -> 30.3 us, E4M3 to FP32 91.9 -> 81.5 us,
            // E4M3 to BF16 unchanged)
            TOut* qp = y + r * ld + b * EPL;
            typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
            if constexpr (sizeof(TOut) == 2) {
                const v4u_t v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                                 pack_bf16x2(o[6], o[7])};
                __builtin_nontemporal_store(v, reinterpret_cast<v4u_t*>(qp));
            } else {
                const v4u_t v0 = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
                const v4u_t v1 = {__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])};
                __builtin_nontemporal_store(v0, reinterpret_cast<v4u_t*>(qp));
                __builtin_nontemporal_store(v1, reinterpret_cast<v4u_t*>(qp) + 1);
            }
        }
    }
}

template <typename T, int ELEM, bool SR>
hipError_t mx_quantize_typed(const T* x, int64_t rows, int64_t cols, int64_t ld, int layout, uint64_t seed,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
    if (layout == kLayoutRow) {
        dim3 g((unsigned)mx_cdiv(cols, 512), mx_grid_y(mx_cdiv(rows, 8)));
        hipLaunchKernelGGL((k_mx_row<T, ELEM, SR>), g, dim3(256), 0, s, x, rows, cols, ld, seed, codes, scales);
    } else {
        dim3 g((unsigned)mx_cdiv(cols, 128 / (int64_t)sizeof(T)), (unsigned)mx_cdiv(rows, 256));
        // nearest-even: runs of tiles along a tile row share one XCD, as for
        // the NVFP4 column tiles (E4M3 8192^2 bf16: 40.0 -> 38.8 us); with
        // stochastic rounding the grouping measured 8% slower
        const int xg = SR ? 1
                       : (g.x % (16 * sizeof(T)) == 0) ? (int)(16 * sizeof(T))
                       : (g.x % (2 * sizeof(T)) == 0) ? (int)(2 * sizeof(T)) : 1;
        hipLaunchKernelGGL((k_mx_col<T, ELEM, SR>), g, dim3(256), 0, s, x, rows, cols, ld, seed, codes, scales,
                           xg);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t mx_quantize_elem(const T* x, int64_t rows, int64_t cols, int64_t ld, int layout, int elem, bool sr,
                            uint64_t seed, uint8_t* codes, uint8_t* scales, hipStream_t s) {
    if (elem == kMxE4M3)
        return sr ? mx_quantize_typed<T, kMxE4M3, true>(x, rows, cols, ld, layout, seed, codes, scales, s)
                  : mx_quantize_typed<T, kMxE4M3, false>(x, rows, cols, ld, layout, seed, codes, scales, s);
    return sr ? mx_quantize_typed<T, kMxE2M1, true>(x, rows, cols, ld, layout, seed, codes, scales, s)
              : mx_quantize_typed<T, kMxE2M1, false>(x, rows, cols, ld, layout, seed, codes, scales, s);
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld, int layout,
                              int elem, bool sr, uint64_t seed, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (bf16)
        return mx_quantize_elem(static_cast<const uint16_t*>(x), rows, cols, ld, layout, elem, sr, seed, codes,
                                scales, s);
    return mx_quantize_elem(static_cast<const float*>(x), rows, cols, ld, layout, elem, sr, seed, codes, scales,
                            s);
}

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int elem, int64_t rows,
                                int64_t cols, void* y, bool bf16, int64_t ld, hipStream_t s) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int wx = cols % 2048 == 0 ? 4 : cols % 1024 == 0 ? 2 : 1;
    dim3 g((unsigned)mx_cdiv(cols / 8, 64 * wx), mx_grid_y(mx_cdiv(rows, 8 * (4 / wx))));
#define NVFP4_MXDQ(E, TO)                                                                                  \
    do {                                                                                                   \
        if (wx == 4)                                                                                       \
            hipLaunchKernelGGL((k_mx_dequant<E, TO, 4>), g, dim3(256), 0, s, codes, scales, rows, cols,   \
                               static_cast<TO*>(y), ld);                                                   \
        else if (wx == 2)                                                                                  \
            hipLaunchKernelGGL((k_mx_dequant<E, TO, 2>), g, dim3(256), 0, s, codes, scales, rows, cols,   \
                               static_cast<TO*>(y), ld);                                                   \
        else                                                                                               \
            hipLaunchKernelGGL((k_mx_dequant<E, TO, 1>), g, dim3(256), 0, s, codes, scales, rows, cols,   \
                               static_cast<TO*>(y), ld);                                                   \
    } while (0)
    if (elem == kMxE4M3) {
        if (bf16) NVFP4_MXDQ(kMxE4M3, uint16_t); else NVFP4_MXDQ(kMxE4M3, float);
    } else {
        if (bf16) NVFP4_MXDQ(kMxE2M1, uint16_t); else NVFP4_MXDQ(kMxE2M1, float);
    }
#undef NVFP4_MXDQ
    return hipGetLastError();
}

}  // namespace nvfp4
