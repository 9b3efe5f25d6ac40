// MX block-scaled GEMM for gfx950 on the scaled matrix cores.
//
// C = A * B^T for A (M x K) and B (N x K) MX tensors with the same element
// format: scaled low-precision products with FP32 accumulation, the block
// scales applied by the hardware ("Nvidia добивается успеха с 4-битным
// форматом NVFP4", asector.ru, section "NVFP4 и Blackwell: интеграция
// архитектуры и формата", describes such block-scaled tensor-core compute;
// MXFP8 is the backward-pass format of "Thinking Machines ускорила обучение
// Inkling 2 Small 4-битными числами", iitak.ru, section "Как это работает").
//
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E4M3 or E2M1 operands
// that carry one E8M0 scale per 32 K elements -- exactly the MX block -- so the
// raw codes and scale bytes go to the matrix core untouched.  Operand layout
// of one 32 x 64 (K) fragment, lane (l, h) = (lane % 32, lane / 32), row l:
//   - E4M3: bytes 0..15 of the 8 dwords hold K = 16 h .. 16 h + 15 (block 0),
//     bytes 16..31 hold K = 32 + 16 h .. (block 1); the lane's scale operand
//     is the scale of block h of its row;
//   - E2M1: dwords 0..3 hold K = 32 h .. 32 h + 31 (block h, low nibble
//     first), dwords 4..7 are unused; scale of block h.
// (Both checked on the hardware against a float64 product; which K a byte
// carries inside a block is immaterial as long as A and B agree, and they
// use the same map.)
//
// Accumulation precision: with E4M3 operands the instruction does not round
// each product sum to binary32: measured against float64 its result is off by
// up to ~2^-12 of the largest product of its 64-element K step (about 13
// significant bits kept while aligning products), where a binary32 sum of
// those products errs by a few units of 2^-24.  E2M1 products (at most 4
// significant bits, small exponent spread) come out exact.  The tolerance of
// the parity tests follows from this measured behaviour.
//
// Geometry and pipeline: a 256-thread workgroup owns a 256 x 256 output tile,
// its four waves a 2 x 2 grid of 128 x 128 wave tiles (4 x 4 MFMAs per 64-wide
// K step).  Raw codes and scale bytes of both operands travel from global
// memory to LDS by global_load_lds (lane i of a load lands at base + size i)
// into a ring of four slots, four steps ahead of use (a row's two scale bytes
// of a step land in one LDS dword, as sub-dword loads do).  Each slot row holds one
// step of one operand row (64 bytes E4M3, 32 bytes E2M1) in 16-byte chunks
// placed at chunk c ^ swz(row), so the fragment reads (ds_read_b128, one row
// per lane) touch every bank once per 8 or 16 lanes; the loads realise the
// swizzle by choosing each lane's source chunk.  Per step and wave: 8 MFMAs,
// then wait for the wave's own loads of the next step, the workgroup barrier,
// the fragment reads of the next step (into the other register set) and the
// loads of the step four ahead into the slot just released, then the other 8
// MFMAs.  The step count is padded to even with a leading step of zero
// operands, so the two register sets alternate statically.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void gmem_t;
typedef __attribute__((address_space(3))) void lmem_t;

constexpr int kMxTile = 256;  // tile rows of A and of B
constexpr int kMxStepK = 64;  // K elements per step (one MFMA K)
constexpr int kMxRing = 4;

template <int ELEM>
struct MxGeo {
    static constexpr int RB = ELEM == kMxE4M3 ? 64 : 32;  // code bytes of a row per step
    static constexpr int CPR = RB / 16;                   // 16-byte chunks per row
    static constexpr int RPL = 1024 / RB;                 // rows per wave-wide 16-byte load
    static constexpr int LOADS = 64 / RPL;                // code loads per operand per wave
    static constexpr int CODES = kMxTile * RB;            // code bytes per operand per slot
    static constexpr int SC = kMxTile * 4;                // scale area per operand per slot (4 bytes a row)
    static constexpr int SLOT = 2 * CODES + 2 * SC;
    static constexpr int LPS = 2 * LOADS + 2;             // loads per wave per step
    static constexpr int FMT = ELEM == kMxE4M3 ? 0 : 4;   // matrix-core operand format
};

// Physical chunk of logical chunk c in slot row r.  E4M3 (4 chunks): the 8
// rows of any 8 consecutive lanes, and the 16 rows of any 16, fall on distinct
// (row bank offset, chunk) pairs; E2M1 (2 chunks) likewise.
template <int CPR>
__device__ __forceinline__ int mx_chunk(int r, int c) {
    return CPR == 4 ? c ^ (((r >> 1) ^ (r >> 3)) & 3) : c ^ (((r >> 2) ^ (r >> 3)) & 1);
}

struct MxGemmArgs {
    const uint8_t *ac, *as, *bc, *bs;
    int64_t M, N, K;
    void* C;
    int64_t ldc;
};

template <int ELEM>
struct MxSrc {
    const uint8_t* a[MxGeo<ELEM>::LOADS];
    const uint8_t* b[MxGeo<ELEM>::LOADS];
    const uint8_t *as, *bs;
};

template <int ELEM>
__device__ __forceinline__ void mx_ring_load(const MxSrc<ELEM>& src, int64_t kc, uint8_t* slot, int w) {
    using G = MxGeo<ELEM>;
    const int64_t co = kc * G::RB, so = kc * 2;
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t)
        __builtin_amdgcn_global_load_lds((gmem_t*)(src.a[t] + co), (lmem_t*)(slot + (64 * w + G::RPL * t) * G::RB),
                                         16, 0, 0);
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t)
        __builtin_amdgcn_global_load_lds((gmem_t*)(src.b[t] + co),
                                         (lmem_t*)(slot + G::CODES + (64 * w + G::RPL * t) * G::RB), 16, 0, 0);
    // a 1- or 2-byte global_load_lds writes lane i's data zero-extended into
    // the dword at base + 4 i, so each row's two scale bytes take a dword
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.as + so), (lmem_t*)(slot + 2 * G::CODES + 256 * w), 2, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.bs + so), (lmem_t*)(slot + 2 * G::CODES + G::SC + 256 * w), 2,
                                     0, 0);
}

// s_waitcnt immediate (gfx9 encoding): at most n vector memory operations of
// this wave outstanding, other counters untouched.
constexpr unsigned mx_vmcnt_at_most(unsigned n) {
    return (n & 15u) | ((n >> 4) << 14) | (7u << 4) | (15u << 8);
}

struct MxFrags {
    v8i_t a[4], b[4];
    int sa[4], sb[4];
};

// Fragment of slot row r (operand base `ops`) for lane half h.
template <int ELEM>
__device__ __forceinline__ v8i_t mx_frag(const uint8_t* ops, int r, int h) {
    using G = MxGeo<ELEM>;
    const uint8_t* row = ops + r * G::RB;
    const uint4 lo = *reinterpret_cast<const uint4*>(row + 16 * mx_chunk<G::CPR>(r, h));
    v8i_t v;
    v[0] = (int)lo.x;
    v[1] = (int)lo.y;
    v[2] = (int)lo.z;
    v[3] = (int)lo.w;
    if constexpr (ELEM == kMxE4M3) {
        const uint4 hi = *reinterpret_cast<const uint4*>(row + 16 * mx_chunk<G::CPR>(r, 2 + h));
        v[4] = (int)hi.x;
        v[5] = (int)hi.y;
        v[6] = (int)hi.z;
        v[7] = (int)hi.w;
    } else {
        v[4] = v[5] = v[6] = v[7] = 0;
    }
    return v;
}

template <int ELEM>
__device__ __forceinline__ void mx_read_frags(const uint8_t* slot, int arow0, int brow0, int l32, int h, bool zero,
                                              MxFrags& f) {
    using G = MxGeo<ELEM>;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = arow0 + 32 * i + l32, rb = brow0 + 32 * i + l32;
        f.a[i] = mx_frag<ELEM>(slot, ra, h);
        f.b[i] = mx_frag<ELEM>(slot + G::CODES, rb, h);
        f.sa[i] = slot[2 * G::CODES + 4 * ra + h];
        f.sb[i] = slot[2 * G::CODES + G::SC + 4 * rb + h];
    }
    if (zero) {  // a padding step: zero A operands make every product 0
#pragma unroll
        for (int i = 0; i < 4; ++i) f.a[i] = v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
}

template <int ELEM, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1) k_mx_gemm(MxGemmArgs p) {
    using G = MxGeo<ELEM>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kMxRing * G::SLOT];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = (int64_t)blockIdx.y * kMxTile, n0 = (int64_t)blockIdx.x * kMxTile;
    const int64_t kb = ELEM == kMxE4M3 ? K : K / 2, ks = K / 32;

    // per-lane sources (rows past the end are clamped re-reads, never stored)
    MxSrc<ELEM> src;
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t) {
        const int r = 64 * w + G::RPL * t + lane / G::CPR;
        const int c = mx_chunk<G::CPR>(r, lane % G::CPR);  // the swizzle is an involution
        src.a[t] = p.ac + min(m0 + r, M - 1) * kb + 16 * c;
        src.b[t] = p.bc + min(n0 + r, N - 1) * kb + 16 * c;
    }
    src.as = p.as + min(m0 + 64 * w + lane, M - 1) * ks;
    src.bs = p.bs + min(n0 + 64 * w + lane, N - 1) * ks;

    v16f_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int arow0 = 128 * wm, brow0 = 128 * wn;
    const int64_t nsteps = K / kMxStepK;
    if (nsteps > 0) {
        const int64_t pad = nsteps & 1, nj = nsteps + pad, last = nsteps - 1;
        auto kc_of = [&](int64_t j) {
            const int64_t kc = j - pad;
            return kc < 0 ? (int64_t)0 : (kc > last ? last : kc);
        };
#pragma unroll
        for (int j = 0; j < kMxRing; ++j) mx_ring_load<ELEM>(src, kc_of(j), lds + j * G::SLOT, w);
        __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(3 * G::LPS));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        MxFrags fx, fy;
        mx_read_frags<ELEM>(lds, arow0, brow0, l32, h, pad > 0, fx);

        auto step = [&](int64_t j, MxFrags& fc, MxFrags& fn) {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                if (m == 8) {
                    // own loads of step j + 1 landed (j + 2, j + 3 may still be
                    // in flight); after the barrier every wave's part of it is
                    // in LDS and every wave has read step j's slot
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(2 * G::LPS));
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    mx_read_frags<ELEM>(lds + ((j + 1) & 3) * G::SLOT, arow0, brow0, l32, h, j + 1 < pad, fn);
                    mx_ring_load<ELEM>(src, kc_of(j + 4), lds + (j & 3) * G::SLOT, w);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int i = m >> 2, jj = m & 3;
                acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fc.a[i], fc.b[jj], acc[i][jj], G::FMT, G::FMT, 0, fc.sa[i], 0, fc.sb[jj]);
            }
        };
        for (int64_t j = 0; j < nj; j += 2) {
            step(j, fx, fy);
            step(j + 1, fy, fx);
        }
        // the last look-ahead loads (clamped re-reads) land before the
        // workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(0));
    }

    // accumulator r of tile (i, j): row 32 i + 8 (r / 4) + 4 h + r % 4, column
    // 32 j + l32 of the wave tile
    const int64_t mw = m0 + arow0, nw = n0 + brow0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = nw + 32 * j + l32;
            if (c >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = mw + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M) {
                    if (OUT_BF16)
                        static_cast<uint16_t*>(p.C)[m * p.ldc + c] =
                            (uint16_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][r]);
                    else
                        static_cast<float*>(p.C)[m * p.ldc + c] = acc[i][j][r];
                }
            }
        }
}

inline int64_t mx_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int elem, int64_t M, int64_t N, int64_t K, void* C,
                          bool c_bf16, int64_t ldc, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    MxGemmArgs p{a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc};
    dim3 grid((unsigned)mx_cdiv(N, kMxTile), (unsigned)mx_cdiv(M, kMxTile));
#define NVFP4_MXG(E, BF) hipLaunchKernelGGL((k_mx_gemm<E, BF>), grid, dim3(256), 0, s, p)
    if (elem == kMxE4M3) {
        if (c_bf16) NVFP4_MXG(kMxE4M3, true); else NVFP4_MXG(kMxE4M3, false);
    } else {
        if (c_bf16) NVFP4_MXG(kMxE2M1, true); else NVFP4_MXG(kMxE2M1, false);
    }
#undef NVFP4_MXG
    return hipGetLastError();
}

}  // namespace nvfp4
