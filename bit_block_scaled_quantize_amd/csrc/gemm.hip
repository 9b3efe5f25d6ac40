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
// carry an E4M3 multiplier per 16.  So each 16-element block is dequantized
// exactly in registers (E2M1 -> FP16 by byte permutes, times the block
// multiplier with one packed FP16 multiply) and fed to
// v_mfma_f32_32x32x16_f16, accumulating in FP32; the two tensor scales are
// applied once in the epilogue.
//
// Geometry: one wave64 per workgroup owns a 128 x 128 output tile (4 x 4
// MFMA tiles of 32 x 32, 256 FP32 accumulators per lane).  Operands stream
// straight from global memory into registers, 64 K-elements per step: every
// lane loads 16 code bytes (32 elements) and 2 scale bytes per 32-row group.
// Within one 64-wide K step, lanes 0-31 take k in [0, 32) and lanes 32-63
// take k in [32, 64); MFMA step s (0..3) uses k = 32h + 8s .. +7 on lane half
// h.  A and B use the same assignment, so every product pairs equal k.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kTM = 128;   // tile rows (A rows)
constexpr int kTN = 128;   // tile cols (B rows)
constexpr int kBK = 64;    // K elements per step

// E2M1 -> FP16 for 8 codes of one 32-bit word (element j in bits 4j..4j+3),
// returned as 4 words each holding FP16 elements (2j, 2j+1).  Every FP16 value
// of an E2M1 magnitude has a zero low byte, so only the high byte is looked up:
// magnitudes 0..7 -> 0x00 0x38 0x3C 0x3E 0x40 0x42 0x44 0x46 (0, .5, 1, 1.5,
// 2, 3, 4, 6), and the sign bit moves to bit 7 of that byte.
__device__ __forceinline__ void e2m1x8_to_f16(uint32_t w, uint32_t out[4]) {
    const uint32_t lut_lo = 0x3E3C3800u, lut_hi = 0x46444240u;
    uint32_t ev = w & 0x07070707u;
    uint32_t od = (w >> 4) & 0x07070707u;
    uint32_t he = __builtin_amdgcn_perm(lut_hi, lut_lo, ev) | ((w << 4) & 0x80808080u);
    uint32_t ho = __builtin_amdgcn_perm(lut_hi, lut_lo, od) | (w & 0x80808080u);
    out[0] = __builtin_amdgcn_perm(ho, he, 0x040C000Cu);
    out[1] = __builtin_amdgcn_perm(ho, he, 0x050C010Cu);
    out[2] = __builtin_amdgcn_perm(ho, he, 0x060C020Cu);
    out[3] = __builtin_amdgcn_perm(ho, he, 0x070C030Cu);
}

// FP16 pair (both halves) of an E4M3 scale byte (exact).
__device__ __forceinline__ half2_t scale_pair(uint32_t sb) {
    _Float16 h = (_Float16)e4m3_value(sb);
    half2_t r = {h, h};
    return r;
}

// One operand row group: 16 code bytes + 2 scale bytes of a lane for one K step.
struct Frag {
    uint4 codes;
    uint32_t sc;  // scale byte 0 in bits 0..7, byte 1 in bits 8..15
};

// Load the lane's fragment of row `row` for K step kc.  `full` means all 64 K
// elements of the step exist; otherwise only groups below K are read and the
// rest are zero (K % 16 == 0, so a lane's 32 elements are 0, 16 or 32 valid).
__device__ __forceinline__ Frag load_frag(const Operand& op, int64_t row, int64_t K, int64_t kc,
                                          int h, bool full) {
    Frag f;
    const int64_t kel = kc * kBK + 32 * h;          // first K element of the lane
    const uint8_t* cp = op.codes + row * (K / 2) + kel / 2;
    const int64_t kb = kel / 16;                     // first 16-block of the lane
    const uint8_t* sp = op.scale_2d ? op.scales + (row / 16) * (K / 16) + kb
                                    : op.scales + row * (K / 16) + kb;
    if (full) {
        f.codes = *reinterpret_cast<const uint4*>(cp);
        f.sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
    } else {
        const int64_t valid = K - kel;
        f.codes = make_uint4(0u, 0u, 0u, 0u);
        f.sc = 0u;
        if (valid >= 32) {
            f.codes = *reinterpret_cast<const uint4*>(cp);
            f.sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
        } else if (valid >= 16) {
            uint2 c2 = *reinterpret_cast<const uint2*>(cp);
            f.codes.x = c2.x;
            f.codes.y = c2.y;
            f.sc = (uint32_t)sp[0];
        }
    }
    return f;
}

// The 8 FP16 operand values of K sub-step s (k = 32h + 8s .. +7).
__device__ __forceinline__ half8_t frag_operand(const Frag& f, int s) {
    uint32_t w = s == 0 ? f.codes.x : s == 1 ? f.codes.y : s == 2 ? f.codes.z : f.codes.w;
    uint32_t q[4];
    e2m1x8_to_f16(w, q);
    half2_t sc = scale_pair((f.sc >> (8 * (s >> 1))) & 0xFFu);
    half8_t r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        half2_t v = __builtin_bit_cast(half2_t, q[j]) * sc;   // exact product
        r[2 * j] = v[0];
        r[2 * j + 1] = v[1];
    }
    return r;
}

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

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool GROUPED, bool SWIGLU, bool OUT_BF16>
__global__ void __launch_bounds__(64) k_gemm(GemmArgs p) {
    const int lane = threadIdx.x;
    const int h = lane >> 5, l32 = lane & 31;

    // ---- tile -> (rows of A, group) ----
    int64_t m_begin = 0, m_end = p.M, m0;
    int g = 0;
    if (GROUPED) {
        int64_t t = blockIdx.y;
        g = -1;
        for (int gg = 0; gg < p.G; ++gg) {
            int64_t lo = min(max(p.offsets[gg], (int64_t)0), p.M);
            int64_t hi = min(max(p.offsets[gg + 1], lo), p.M);
            int64_t tiles = (hi - lo + kTM - 1) / kTM;
            if (t < tiles) {
                g = gg;
                m_begin = lo;
                m_end = hi;
                m0 = lo + t * kTM;
                break;
            }
            t -= tiles;
        }
        if (g < 0) return;
    } else {
        m0 = (int64_t)blockIdx.y * kTM;
    }
    const int64_t K = p.K;

    // ---- B rows of this tile ----
    // plain / grouped: B rows n0 .. n0+127 of the group's block.
    // SwiGLU: output columns j0 .. j0+63; B rows (gate) j0.. and (up) F + j0..
    int64_t brow[4];
    bool bvalid[4];
    const int64_t Ng = p.N;
    const int64_t bbase = GROUPED ? (int64_t)g * Ng : 0;
    if (SWIGLU) {
        const int64_t F = Ng / 2, j0 = (int64_t)blockIdx.x * (kTN / 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t c = j0 + 32 * (j & 1) + l32;
            bvalid[j] = c < F;
            int64_t r = (j < 2 ? 0 : F) + min(c, F - 1);
            brow[j] = bbase + r;
        }
    } else {
        const int64_t n0 = (int64_t)blockIdx.x * kTN;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t c = n0 + 32 * j + l32;
            bvalid[j] = c < Ng;
            brow[j] = bbase + min(c, Ng - 1);
        }
    }
    int64_t arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) arow[i] = min(m0 + 32 * i + l32, m_end - 1);

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nsteps = (K + kBK - 1) / kBK;
    const int64_t nfull = K / kBK;
    Frag fa[4], fb[4];
    if (nsteps > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = load_frag(p.A, arow[i], K, 0, h, nfull > 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = load_frag(p.B, brow[j], K, 0, h, nfull > 0);
    }
    for (int64_t kc = 0; kc < nsteps; ++kc) {
        Frag na[4], nb[4];
        const bool more = kc + 1 < nsteps;
        if (more) {
            const bool full = kc + 1 < nfull;
#pragma unroll
            for (int i = 0; i < 4; ++i) na[i] = load_frag(p.A, arow[i], K, kc + 1, h, full);
#pragma unroll
            for (int j = 0; j < 4; ++j) nb[j] = load_frag(p.B, brow[j], K, kc + 1, h, full);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8_t bo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) bo[j] = frag_operand(fb[j], s);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                half8_t ao = frag_operand(fa[i], s);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ao, bo[j], acc[i][j], 0, 0, 0);
            }
        }
        if (more) {
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = na[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = nb[j];
        }
    }

    // ---- epilogue ----
    const float alpha = p.A.ts[0] * p.B.ts[GROUPED ? g : 0];
    // accumulator r of tile (i, j): row 32i + 8(r/4) + 4h + r%4, col 32j + l32
    if (SWIGLU) {
        uint16_t* C = static_cast<uint16_t*>(p.C);
        const int64_t F = Ng / 2, j0 = (int64_t)blockIdx.x * (kTN / 2);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int64_t c = j0 + 32 * jj + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (m < m_end && c < F) {
                        float gt = alpha * acc[i][jj][r];
                        float up = alpha * acc[i][jj + 2][r];
                        float hv = gt / (1.0f + expf(-gt)) * up;
                        uint32_t b = f32_to_bf16_rne(hv);
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
    const int64_t n0 = (int64_t)blockIdx.x * kTN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = n0 + 32 * j + l32;
            if (!bvalid[j]) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < m_end) {
                    float v = alpha * acc[i][j][r];
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
    dim3 grid((unsigned)cdiv(N, kTN), (unsigned)cdiv(M, kTM));
    if (c_bf16)
        hipLaunchKernelGGL((k_gemm<false, false, true>), grid, dim3(64), 0, s, p);
    else
        hipLaunchKernelGGL((k_gemm<false, false, false>), grid, dim3(64), 0, s, p);
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
    const int64_t mtiles = cdiv(total_rows, kTM) + G;
    if (swiglu) {
        dim3 grid((unsigned)cdiv(n_per_group / 2, kTN / 2), (unsigned)mtiles);
        hipLaunchKernelGGL((k_gemm<true, true, true>), grid, dim3(64), 0, s, p);
    } else {
        dim3 grid((unsigned)cdiv(n_per_group, kTN), (unsigned)mtiles);
        if (c_bf16)
            hipLaunchKernelGGL((k_gemm<true, false, true>), grid, dim3(64), 0, s, p);
        else
            hipLaunchKernelGGL((k_gemm<true, false, false>), grid, dim3(64), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
