// NVFP4 block-scaled GEMM and grouped (MoE) GEMM for gfx950.
//
// Scaled low-precision compute with high-precision accumulation ("Nvidia
// добивается успеха с 4-битным форматом NVFP4", asector.ru, section "NVFP4 и
// Blackwell: интеграция архитектуры и формата"); grouped over experts as in the
// expert layers' forward pass ("Thinking Machines ускорила обучение Inkling 2
// Small 4-битными числами", iitak.ru, section "Детали").
//
// Why FP16 MFMA: an operand element is v * sb with v an E2M1 value (2
// significant bits) and sb an E4M3 block multiplier (4 significant bits), so
// the product has at most 6 significant bits and lies in [2^-10, 2688].  FP16
// represents every such value exactly; FP8/FP6/FP4 do not, and gfx950's scaled
// FP4 MFMAs take power-of-two (E8M0) scales per 32 elements, which cannot
// carry an E4M3 multiplier per 16.  So every 16-element block is dequantized
// exactly to FP16 and fed to v_mfma_f32_32x32x16_f16 with FP32 accumulation;
// the two tensor scales are applied once in the epilogue.
//
// Geometry: a 256-thread workgroup owns a 256 x 256 output tile; its four
// waves form a 2 x 2 grid of 128 x 128 wave tiles (4 x 4 MFMA tiles of 32 x 32,
// 256 FP32 accumulators per lane).  Each 64-wide K step:
//   1. every thread loads one A row and one B row of the step (32 code bytes +
//      4 scale bytes each) for the NEXT step into registers;
//   2. the waves run the 64 MFMAs of the current step from LDS;
//   3. every thread dequantizes its two prefetched rows to FP16 (FP4 unpack
//      instruction, round-toward-zero pack -- exact here -- and one packed
//      FP16 multiply by the block multiplier) into the other LDS stage;
//   4. one barrier.
// Each operand element is thus expanded once per workgroup instead of once
// per wave that uses it.  LDS: 2 stages x (A, B) x 256 rows x 144 bytes
// (64 FP16 + 16 bytes of padding that spreads the row starts over the banks).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 256;   // tile rows (A rows)
constexpr int kBN = 256;   // tile B rows
constexpr int kBK = 64;    // K elements per step
constexpr int kLdsK = 72;  // FP16 per LDS row (64 + 8 padding)

// Problem description handed to the kernel.
struct GemmArgs {
    Operand A, B;
    int64_t M;              // plain GEMM: rows of A; grouped: total rows
    int64_t N;              // plain: rows of B; grouped: rows per group (2F for SwiGLU)
    int64_t K;
    void* C;
    int64_t ldc;
    const int64_t* offsets; // grouped only
    int G;                  // grouped only
    float* amax_out;        // SwiGLU only, nullable
};

// One row's share of a K step: 64 codes and their four block multipliers.
struct RowStep {
    uint4 c0, c1;  // code bytes 0..15 and 16..31
    uint32_t sc;   // scale bytes of the four 16-element blocks
};

// Load row `row` of operand `op` for K step kc (zeros past K; K % 16 == 0).
__device__ __forceinline__ RowStep load_row_step(const Operand& op, int64_t row, int64_t K,
                                                 int64_t kc, bool full, bool scales_aligned) {
    RowStep r;
    const uint8_t* cp = op.codes + row * (K / 2) + kc * (kBK / 2);
    const int64_t kb = kc * (kBK / 16);
    const uint8_t* sp = op.scale_2d ? op.scales + (row / 16) * (K / 16) + kb
                                    : op.scales + row * (K / 16) + kb;
    if (full) {
        r.c0 = *reinterpret_cast<const uint4*>(cp);
        r.c1 = *reinterpret_cast<const uint4*>(cp + 16);
        r.sc = scales_aligned ? *reinterpret_cast<const uint32_t*>(sp)
                              : (uint32_t)sp[0] | ((uint32_t)sp[1] << 8) | ((uint32_t)sp[2] << 16) |
                                    ((uint32_t)sp[3] << 24);
    } else {
        const int64_t nblk = (K - kc * kBK) / 16;  // 1..3 valid 16-element blocks
        r.c0 = make_uint4(0u, 0u, 0u, 0u);
        r.c1 = make_uint4(0u, 0u, 0u, 0u);
        r.sc = 0u;
        const uint2* c2 = reinterpret_cast<const uint2*>(cp);
        if (nblk > 0) { uint2 t = c2[0]; r.c0.x = t.x; r.c0.y = t.y; r.sc = sp[0]; }
        if (nblk > 1) { uint2 t = c2[1]; r.c0.z = t.x; r.c0.w = t.y; r.sc |= (uint32_t)sp[1] << 8; }
        if (nblk > 2) { uint2 t = c2[2]; r.c1.x = t.x; r.c1.y = t.y; r.sc |= (uint32_t)sp[2] << 16; }
    }
    return r;
}

// 8 codes (one 32-bit word) -> 8 FP16 values times the block multiplier,
// returned as 4 words of FP16 pairs.  Exact throughout: the unpack gives the
// E2M1 values in binary32, the round-toward-zero FP16 pack keeps them (2
// significant bits), and their products with an E4M3 value have at most 6.
__device__ __forceinline__ uint4 dequant8_f16(uint32_t w, half2_t sc) {
    uint32_t q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float2 f = e2m1x2_unpack(w, k);
        half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(f.x, f.y));
        q[k] = __builtin_bit_cast(uint32_t, h * sc);
    }
    return make_uint4(q[0], q[1], q[2], q[3]);
}

__device__ __forceinline__ half2_t scale_pair(uint32_t sb) {
    _Float16 h = (_Float16)e4m3_value(sb);
    half2_t r = {h, h};
    return r;
}

// Dequantize one RowStep into LDS row `dst` (64 FP16, natural K order).
__device__ __forceinline__ void store_row_step(const RowStep& r, _Float16* dst) {
    const uint32_t w[8] = {r.c0.x, r.c0.y, r.c0.z, r.c0.w, r.c1.x, r.c1.y, r.c1.z, r.c1.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const half2_t sc = scale_pair((r.sc >> (8 * q)) & 0xFFu);
        *reinterpret_cast<uint4*>(dst + 16 * q) = dequant8_f16(w[2 * q], sc);
        *reinterpret_cast<uint4*>(dst + 16 * q + 8) = dequant8_f16(w[2 * q + 1], sc);
    }
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

template <bool GROUPED, bool SWIGLU, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1) k_gemm(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) _Float16 smem[2][2][kBM][kLdsK];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;

    // ---- tile -> (rows of A, group) ----
    int64_t m_end = p.M, m0 = 0;
    int g = 0;
    if (GROUPED) {
        int64_t t = blockIdx.y;
        g = -1;
        for (int gg = 0; gg < p.G; ++gg) {
            const int64_t lo = min(max(p.offsets[gg], (int64_t)0), p.M);
            const int64_t hi = min(max(p.offsets[gg + 1], lo), p.M);
            const int64_t tiles = (hi - lo + kBM - 1) / kBM;
            if (t < tiles) {
                g = gg;
                m_end = hi;
                m0 = lo + t * kBM;
                break;
            }
            t -= tiles;
        }
        if (g < 0) return;  // uniform across the workgroup
    } else {
        m0 = (int64_t)blockIdx.y * kBM;
    }
    const int64_t K = p.K, Ng = p.N;
    const int64_t bbase = GROUPED ? (int64_t)g * Ng : 0;

    // ---- the A row and B row this thread stages ----
    const int64_t arow = min(m0 + tid, m_end - 1);
    int64_t brow;
    if (SWIGLU) {
        const int64_t F = Ng / 2, j0 = (int64_t)blockIdx.x * (kBN / 2);
        const int64_t c = min(j0 + (tid & 127), F - 1);
        brow = bbase + (tid < 128 ? c : F + c);
    } else {
        brow = bbase + min((int64_t)blockIdx.x * kBN + tid, Ng - 1);
    }

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nsteps = (K + kBK - 1) / kBK;
    const int64_t nfull = K / kBK;
    // 4-byte scale loads when every step's four scale bytes are 4-byte aligned
    const bool sal_a = (K % kBK) == 0 && (reinterpret_cast<uintptr_t>(p.A.scales) & 3) == 0;
    const bool sal_b = (K % kBK) == 0 && (reinterpret_cast<uintptr_t>(p.B.scales) & 3) == 0;

    // LDS rows read by this wave's MFMA tiles (A: 4 tiles of 32 rows; B likewise)
    int brow_lds[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        brow_lds[j] = SWIGLU ? ((j < 2 ? 0 : 128) + 64 * wn + 32 * (j & 1)) : 128 * wn + 32 * j;

    if (nsteps > 0) {
        RowStep ra = load_row_step(p.A, arow, K, 0, nfull > 0, sal_a);
        RowStep rb = load_row_step(p.B, brow, K, 0, nfull > 0, sal_b);
        store_row_step(ra, &smem[0][0][tid][0]);
        store_row_step(rb, &smem[0][1][tid][0]);
    }
    __syncthreads();

    for (int64_t kc = 0; kc < nsteps; ++kc) {
        const int st = (int)(kc & 1);
        const bool more = kc + 1 < nsteps;
        RowStep na, nb;
        if (more) {
            const bool full = kc + 1 < nfull;
            na = load_row_step(p.A, arow, K, kc + 1, full, sal_a);
            nb = load_row_step(p.B, brow, K, kc + 1, full, sal_b);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8_t bo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bo[j] = *reinterpret_cast<const half8_t*>(&smem[st][1][brow_lds[j] + l32][16 * s + 8 * h]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half8_t ao =
                    *reinterpret_cast<const half8_t*>(&smem[st][0][128 * wm + 32 * i + l32][16 * s + 8 * h]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao, bo[j], acc[i][j], 0, 0, 0);
            }
        }
        if (more) {
            store_row_step(na, &smem[st ^ 1][0][tid][0]);
            store_row_step(nb, &smem[st ^ 1][1][tid][0]);
        }
        __syncthreads();
    }

    // ---- epilogue ----
    const float alpha = p.A.ts[0] * p.B.ts[GROUPED ? g : 0];
    // accumulator r of MFMA tile (i, j): row 32i + 8(r/4) + 4h + r%4, col 32j + l32
    const int64_t mw = m0 + 128 * wm;
    if (SWIGLU) {
        uint16_t* C = static_cast<uint16_t*>(p.C);
        const int64_t F = Ng / 2, jw = (int64_t)blockIdx.x * (kBN / 2) + 64 * wn;
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int64_t c = jw + 32 * jj + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = mw + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (m < m_end && c < F) {
                        const float gt = alpha * acc[i][jj][r];
                        const float up = alpha * acc[i][jj + 2][r];
                        const float hv = gt / (1.0f + expf(-gt)) * up;
                        const uint32_t b = f32_to_bf16_rne(hv);
                        C[m * p.ldc + c] = (uint16_t)b;
                        amax = fmaxf(amax, fabsf(__uint_as_float(b << 16)));
                    }
                }
            }
        if (p.amax_out) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(p.amax_out), __float_as_uint(amax));
        }
        return;
    }
    const int64_t nw = (int64_t)blockIdx.x * kBN + 128 * wn;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = nw + 32 * j + l32;
            if (c >= Ng) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = mw + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < m_end) {
                    const float v = alpha * acc[i][j][r];
                    if (OUT_BF16)
                        static_cast<uint16_t*>(p.C)[m * p.ldc + c] = (uint16_t)f32_to_bf16_rne(v);
                    else
                        static_cast<float*>(p.C)[m * p.ldc + c] = v;
                }
            }
        }
}

__global__ void k_zero_float(float* p) {
    if (threadIdx.x == 0) p[0] = 0.0f;
}

namespace {
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

hipError_t launch_gemm(const Operand& A, const Operand& B, int64_t M, int64_t N, int64_t K,
                       void* C, bool c_bf16, int64_t ldc, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    GemmArgs p{A, B, M, N, K, C, ldc, nullptr, 1, nullptr};
    dim3 grid((unsigned)cdiv(N, kBN), (unsigned)cdiv(M, kBM));
    if (c_bf16)
        hipLaunchKernelGGL((k_gemm<false, false, true>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((k_gemm<false, false, false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(int G, const Operand& A, const int64_t* offsets, int64_t total_rows,
                               const Operand& B, int64_t n_per_group, int64_t K, void* C,
                               bool c_bf16, int64_t ldc, bool swiglu, float* amax_out,
                               hipStream_t s) {
    if (swiglu && amax_out) hipLaunchKernelGGL(k_zero_float, dim3(1), dim3(64), 0, s, amax_out);
    if (total_rows == 0 || n_per_group == 0) return hipGetLastError();
    GemmArgs p{A, B, total_rows, n_per_group, K, C, ldc, offsets, G, amax_out};
    // every group wastes at most one partial tile
    const int64_t mtiles = cdiv(total_rows, kBM) + G;
    if (swiglu) {
        dim3 grid((unsigned)cdiv(n_per_group / 2, kBN / 2), (unsigned)mtiles);
        hipLaunchKernelGGL((k_gemm<true, true, true>), grid, dim3(256), 0, s, p);
    } else {
        dim3 grid((unsigned)cdiv(n_per_group, kBN), (unsigned)mtiles);
        if (c_bf16)
            hipLaunchKernelGGL((k_gemm<true, false, true>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((k_gemm<true, false, false>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
