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
// Ring kernel (any K % 64 == 0; the full-line kernel further down serves
// K % 1024 == 0): a 256-thread workgroup owns a 256 x 256 output tile,
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
// MFMAs.  The step count is padded to a multiple of 4 with leading steps whose
// slots are zero-filled, so slots and register sets have static names and the
// loop body has no branch.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace nvfp4 {

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef int v4i_t __attribute__((ext_vector_type(4)));

// 16 bytes of LDS as one vector load (one ds_read_b128 that keeps the
// access's memory information; a struct load is split into dwords and
// re-merged, and the compiler then lost track of which slot a read touches
// and waited for every outstanding load before it).
__device__ __forceinline__ v4i_t lds16(const uint8_t* p) { return *reinterpret_cast<const v4i_t*>(p); }
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(1))) void gmem_t;
typedef __attribute__((address_space(3))) void lmem_t;

constexpr int kMxTile = 256;  // tile rows of A and of B
constexpr int kMxStepK = 64;  // K elements per step (one MFMA K)

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

// Physical chunk of logical chunk c in slot row r (a function of row bits
// 1..4 only).  E4M3 (4 chunks): the 8 rows of any 8 consecutive lanes, and the
// 16 rows of any 16, fall on distinct (row bank offset, chunk) pairs; E2M1 (2
// chunks) likewise.
template <int CPR>
__device__ __forceinline__ int mx_chunk(int r, int c) {
    return CPR == 4 ? c ^ (((r >> 1) ^ (r >> 3)) & 3) : c ^ (((r >> 2) ^ (r >> 3)) & 1);
}

struct MxGemmArgs {
    const uint8_t *ac, *as, *bc, *bs;
    int64_t M, N, K;
    void* C;
    int64_t ldc;
    // full-line native kernel only (one-dimensional grid): tiles row-major
    // over a tiles_x-wide grid; those from t_main on split `split` ways along
    // K, their parts' binary32 sums written as 256 x 256 matrices to `parts`
    int tiles_x, t_main, split;
    float* parts;
    int first;  // work item of workgroup 0 (a launch of parts only starts past the whole tiles)
};

// Global sources of a workgroup's ring loads: wave-uniform bases (the tile's
// first A and B rows) and 32-bit per-lane byte offsets from them (the tile
// spans 256 rows, so offsets stay below 256 row lengths).
template <int ELEM>
struct MxSrc {
    const uint8_t *ac, *bc, *as, *bs;
    uint32_t a[MxGeo<ELEM>::LOADS];
    uint32_t b[MxGeo<ELEM>::LOADS];
    uint32_t sa, sb;
};

template <int ELEM>
__device__ __forceinline__ void mx_ring_load(const MxSrc<ELEM>& src, int64_t kc, uint8_t* slot, int w) {
    using G = MxGeo<ELEM>;
    const uint8_t* ac = src.ac + kc * G::RB;
    const uint8_t* bc = src.bc + kc * G::RB;
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t)
        __builtin_amdgcn_global_load_lds((gmem_t*)(ac + src.a[t]), (lmem_t*)(slot + (64 * w + G::RPL * t) * G::RB),
                                         16, 0, 0);
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t)
        __builtin_amdgcn_global_load_lds((gmem_t*)(bc + src.b[t]),
                                         (lmem_t*)(slot + G::CODES + (64 * w + G::RPL * t) * G::RB), 16, 0, 0);
    // a 1- or 2-byte global_load_lds writes lane i's data zero-extended into
    // the dword at base + 4 i, so each row's two scale bytes take a dword
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.as + 2 * kc + src.sa), (lmem_t*)(slot + 2 * G::CODES + 256 * w),
                                     2, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.bs + 2 * kc + src.sb),
                                     (lmem_t*)(slot + 2 * G::CODES + G::SC + 256 * w), 2, 0, 0);
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

// A lane's byte offsets inside a slot for its fragment rows of MFMA tile 0
// (rows arow0 + l32 of A and brow0 + l32 of B): codes of its two chunks per
// operand and its scale byte.  Tile i adds 32 i rows, which leaves the chunk
// swizzle unchanged (it depends on row bits 1..4 only), so every fragment
// read is one of these offsets plus a compile-time constant.
struct MxLaneOffsets {
    int a_lo, a_hi, b_lo, b_hi, sa, sb;
};

template <int ELEM>
__device__ __forceinline__ MxLaneOffsets mx_lane_offsets(int arow0, int brow0, int l32, int h) {
    using G = MxGeo<ELEM>;
    MxLaneOffsets o;
    const int ra = arow0 + l32, rb = brow0 + l32;
    o.a_lo = ra * G::RB + 16 * mx_chunk<G::CPR>(l32, h);
    o.b_lo = G::CODES + rb * G::RB + 16 * mx_chunk<G::CPR>(l32, h);
    o.a_hi = ra * G::RB + 16 * mx_chunk<G::CPR>(l32, (2 + h) & (G::CPR - 1));
    o.b_hi = G::CODES + rb * G::RB + 16 * mx_chunk<G::CPR>(l32, (2 + h) & (G::CPR - 1));
    o.sa = 2 * G::CODES + 4 * ra + h;
    o.sb = 2 * G::CODES + G::SC + 4 * rb + h;
    return o;
}

template <int ELEM>
__device__ __forceinline__ v8i_t mx_frag(const uint8_t* slot, int lo, int hi) {
    const uint4 q = *reinterpret_cast<const uint4*>(slot + lo);
    v8i_t v;
    v[0] = (int)q.x;
    v[1] = (int)q.y;
    v[2] = (int)q.z;
    v[3] = (int)q.w;
    if constexpr (ELEM == kMxE4M3) {
        const uint4 r = *reinterpret_cast<const uint4*>(slot + hi);
        v[4] = (int)r.x;
        v[5] = (int)r.y;
        v[6] = (int)r.z;
        v[7] = (int)r.w;
    } else {
        v[4] = v[5] = v[6] = v[7] = 0;
    }
    return v;
}

template <int ELEM>
__device__ __forceinline__ void mx_read_frags(const uint8_t* slot, const MxLaneOffsets& o, MxFrags& f) {
    using G = MxGeo<ELEM>;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dc = 32 * i * G::RB, ds = 32 * i * 4;
        f.a[i] = mx_frag<ELEM>(slot + dc, o.a_lo, o.a_hi);
        f.b[i] = mx_frag<ELEM>(slot + dc, o.b_lo, o.b_hi);
        f.sa[i] = slot[o.sa + ds];
        f.sb[i] = slot[o.sb + ds];
    }
}

// A padding step's slot, all of it set to zero (codes +0, scale bytes 2^-127:
// every product of the step is +0; leaving the B half or the scale bytes
// uninitialized could pair a zero with a NaN pattern), written by the whole
// workgroup.
template <int ELEM>
__device__ __forceinline__ void mx_zero_slot(uint8_t* slot) {
    using G = MxGeo<ELEM>;
    static_assert((2 * G::CODES) % (256 * 16) == 0 && 2 * G::SC == 256 * 8, "zero-fill geometry");
    // codes of A and B occupy [0, 2 CODES): 16-byte stores; scale bytes
    // [2 CODES, 2 CODES + 2 SC): 8 bytes per thread
#pragma unroll
    for (int k = 0; k < 2 * G::CODES / (256 * 16); ++k)
        *reinterpret_cast<uint4*>(slot + 16 * (threadIdx.x + 256 * k)) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint2*>(slot + 2 * G::CODES + 8 * threadIdx.x) = make_uint2(0u, 0u);
}

// s_waitcnt immediate: all LDS operations of this wave done, vector memory
// and export counters untouched.
constexpr unsigned mx_lgkmcnt_zero() { return 15u | (3u << 14) | (7u << 4); }

template <int ELEM, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1) k_mx_gemm(MxGemmArgs p) {
    using G = MxGeo<ELEM>;
    // four slots as four variables: the compiler then sees that a slot being
    // read is not one that in-flight global_load_lds writes target, and waits
    // only where the code says so (one shared array makes it wait for every
    // outstanding load before each LDS read)
    __shared__ __attribute__((aligned(16))) uint8_t ring0[G::SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[G::SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[G::SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[G::SLOT];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = (int64_t)blockIdx.y * kMxTile, n0 = (int64_t)blockIdx.x * kMxTile;
    const int64_t kb = ELEM == kMxE4M3 ? K : K / 2, ks = K / 32;

    // per-lane sources (rows past the end are clamped re-reads, never stored)
    MxSrc<ELEM> src;
    src.ac = p.ac + m0 * kb;
    src.bc = p.bc + n0 * kb;
    src.as = p.as + m0 * ks;
    src.bs = p.bs + n0 * ks;
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t) {
        const int r = 64 * w + G::RPL * t + lane / G::CPR;
        const int c = mx_chunk<G::CPR>(r, lane % G::CPR);  // the swizzle is an involution
        src.a[t] = (uint32_t)((min(m0 + r, M - 1) - m0) * kb + 16 * c);
        src.b[t] = (uint32_t)((min(n0 + r, N - 1) - n0) * kb + 16 * c);
    }
    src.sa = (uint32_t)((min(m0 + 64 * w + lane, M - 1) - m0) * ks);
    src.sb = (uint32_t)((min(n0 + 64 * w + lane, N - 1) - n0) * ks);

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
        // steps run four at a time (static slot names); the count is padded to
        // a multiple of 4 with leading steps whose slots hold zeros
        // (filled once here: the loop itself has no branch, so the compiler
        // keeps each step's MFMAs between its barriers)
        const int64_t pad = (4 - nsteps % 4) % 4, nj = nsteps + pad, last = nsteps - 1;
        // (a padding slot is never reloaded before its step has been read)
        auto kc_of = [&](int64_t j) {
            const int64_t kc = j - pad;
            return kc < 0 ? (int64_t)0 : (kc > last ? last : kc);
        };
        if (pad > 0) mx_zero_slot<ELEM>(ring0); else mx_ring_load<ELEM>(src, kc_of(0), ring0, w);
        if (pad > 1) mx_zero_slot<ELEM>(ring1); else mx_ring_load<ELEM>(src, kc_of(1), ring1, w);
        if (pad > 2) mx_zero_slot<ELEM>(ring2); else mx_ring_load<ELEM>(src, kc_of(2), ring2, w);
        mx_ring_load<ELEM>(src, kc_of(3), ring3, w);
        // step 0 landed (pads come first, so if step 0 is loaded so are 1..3)
        // and the zero fills done, then the barrier
        __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(3 * G::LPS));
        __builtin_amdgcn_s_waitcnt(mx_lgkmcnt_zero());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        const MxLaneOffsets lo = mx_lane_offsets<ELEM>(arow0, brow0, l32, h);
        MxFrags fx, fy;
        mx_read_frags<ELEM>(ring0, lo, fx);

        auto step = [&](int64_t j, uint8_t* cur, uint8_t* nxt, MxFrags& fc, MxFrags& fn) {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                if (m == 8) {
                    // own loads of step j + 1 landed (j + 2, j + 3 may still be
                    // in flight; a padding step j + 1 loaded nothing and so
                    // needs no wait); after the barrier every wave's part of
                    // it is in LDS and every wave has read step j's slot
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(2 * G::LPS));
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    mx_read_frags<ELEM>(nxt, lo, fn);
                    mx_ring_load<ELEM>(src, kc_of(j + 4), cur, w);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int i = m >> 2, jj = m & 3;
                acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fc.a[i], fc.b[jj], acc[i][jj], G::FMT, G::FMT, 0, fc.sa[i], 0, fc.sb[jj]);
            }
        };
        for (int64_t j = 0; j < nj; j += 4) {
            step(j, ring0, ring1, fx, fy);
            step(j + 1, ring1, ring2, fy, fx);
            step(j + 2, ring2, ring3, fx, fy);
            step(j + 3, ring3, ring0, fy, fx);
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

// ============================================================ exact accumulation
// For callers that need the NVFP4 GEMM's accuracy (|C - exact| within
// 1e-5 sum |a b|) from MX operands: the scaled matrix core keeps only ~13 bits
// while it sums a K step of E4M3 products, so here every element is converted
// exactly to BF16 and the BF16 matrix core (v_mfma_f32_32x32x16_bf16) forms
// exact products and sums them in binary32, as the NVFP4 GEMM does in FP16.
// BF16 keeps binary32's 8 exponent bits, so an element carries its block
// scale as a power of two relative to the largest block scale of its row:
// A'[m][k] = v * 2^(b[m][kb] - R[m]), R[m] = max over kb of the scale byte
// b[m][kb]; then C[m][n] = 2^(R_A[m] + R_B[n] - 254) * sum_k A'[m][k] B'[n][k]
// (E8M0 bytes carry a bias of 127).  One gfx950 scaled convert
// (v_cvt_scalef32_pk_bf16_fp8 / _fp4) turns two codes into two BF16 values
// times that power of two; its f32 scale operand contributes its exponent
// only, so the operand is built as 2^e directly.  Every product is exact while
// the rescaled elements and their products stay in the normal ranges of BF16
// and binary32: a nonzero E4M3 element is at least 2^-9 (E2M1: 2^-1), so it
// suffices that for each block the two rows' distances below their largest
// scales add up to at most 108 binades (E2M1: 124) -- e.g. every row's
// nonzero blocks within 2^54 of its largest.  A block more than 2^126 below
// is scaled by 2^-126 (a clamp that keeps the operand a normal binary32).
//
// Pipeline: the ring kernel's (four 64-step slots of raw codes and scale
// bytes, loaded by global_load_lds three steps ahead, one barrier per step),
// with each 64-wide K step run as four 16-wide substeps of 16 BF16 MFMAs per
// wave; a lane converts its 8 elements of each fragment for the substep just
// before its MFMAs.  Substep q takes bytes 8q .. 8q+7 of the lane's E4M3
// fragment (block q / 2 of the step) or nibbles 8q .. 8q+7 of its E2M1
// fragment (block h); A and B use the same map, so the products pair the
// same K.  The largest scale byte of each tile row is found once, in the
// prologue, from the rows' scale bytes.
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));

// Largest byte of p[0 .. n).
__device__ __forceinline__ int row_max_byte(const uint8_t* p, int64_t n) {
    uint32_t m = 0u;
    int64_t k = 0;
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
        for (; k + 16 <= n; k += 16) {
            const uint4 v = *reinterpret_cast<const uint4*>(p + k);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int d = 0; d < 4; ++d)
                m = max(m, max(max(w[d] & 0xFFu, (w[d] >> 8) & 0xFFu), max((w[d] >> 16) & 0xFFu, w[d] >> 24)));
        }
    }
    for (; k < n; ++k) m = max(m, (uint32_t)p[k]);
    return (int)m;
}

// 2^(b - r) as a binary32 scale operand (b <= r), at least 2^-126.
__device__ __forceinline__ float pow2_rel(int b, int r) {
    return __uint_as_float((uint32_t)(127 + max(b - r, -126)) << 23);
}

// The lane's 8 elements of substep q of its fragment f, as BF16 times sc.
template <int ELEM>
__device__ __forceinline__ v8bf_t exact_piece(const v8i_t& f, int q, float sc) {
    v2bf_t p0, p1, p2, p3;
    if constexpr (ELEM == kMxE4M3) {
        const uint32_t d0 = (uint32_t)f[2 * q], d1 = (uint32_t)f[2 * q + 1];
        p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, false);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, sc, true);
        p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, false);
        p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, sc, true);
    } else {
        const uint32_t d = (uint32_t)f[q];
        p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0);
        p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1);
        p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2);
        p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3);
    }
    return v8bf_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Raw fragments of a step (as mx_read_frags) with the scale bytes an exact
// conversion needs: E4M3 lanes hold elements of both blocks of the step (the
// row's two bytes, block 0 in bits 0..7), E2M1 lanes of block h only.
template <int ELEM>
__device__ __forceinline__ void mx_read_frags_exact(const uint8_t* slot, const MxLaneOffsets& o, MxFrags& f) {
    using G = MxGeo<ELEM>;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int dc = 32 * i * G::RB, ds = 32 * i * 4;
        f.a[i] = mx_frag<ELEM>(slot + dc, o.a_lo, o.a_hi);
        f.b[i] = mx_frag<ELEM>(slot + dc, o.b_lo, o.b_hi);
        if constexpr (ELEM == kMxE4M3) {
            // o.sa - h is the row's dword: bytes 0 and 1 are blocks 0 and 1
            f.sa[i] = *reinterpret_cast<const uint16_t*>(slot + o.sa - (o.sa & 3) + ds);
            f.sb[i] = *reinterpret_cast<const uint16_t*>(slot + o.sb - (o.sb & 3) + ds);
        } else {
            f.sa[i] = slot[o.sa + ds];
            f.sb[i] = slot[o.sb + ds];
        }
    }
}

// Fragment o (0..3: A tile o, 4..7: B tile o - 4) of mx_read_frags_exact, on
// its own.
template <int ELEM>
__device__ __forceinline__ void mx_read_frag_exact(const uint8_t* slot, const MxLaneOffsets& lo, int o, MxFrags& f) {
    using G = MxGeo<ELEM>;
    const bool isb = o >= 4;
    const int i = isb ? o - 4 : o;
    const int dc = 32 * i * G::RB, ds = 32 * i * 4;
    const v8i_t v = mx_frag<ELEM>(slot + dc, isb ? lo.b_lo : lo.a_lo, isb ? lo.b_hi : lo.a_hi);
    const int so = isb ? lo.sb : lo.sa;
    int sc;
    if constexpr (ELEM == kMxE4M3) sc = *reinterpret_cast<const uint16_t*>(slot + so - (so & 3) + ds);
    else sc = slot[so + ds];
    if (isb) {
        f.b[i] = v;
        f.sb[i] = sc;
    } else {
        f.a[i] = v;
        f.sa[i] = sc;
    }
}

// Pair pr (0..3) of substep q of fragment f as two BF16 values times sc (the
// pairs of exact_piece, one convert each).
template <int ELEM>
__device__ __forceinline__ uint32_t exact_pair(const v8i_t& f, int q, int pr, float sc) {
    v2bf_t v;
    if constexpr (ELEM == kMxE4M3) {
        const uint32_t d = (uint32_t)f[2 * q + (pr >> 1)];
        v = (pr & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, sc, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, sc, false);
    } else {
        const uint32_t d = (uint32_t)f[q];
        switch (pr) {
            case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0); break;
            case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1); break;
            case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2); break;
            default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3); break;
        }
    }
    return __builtin_bit_cast(uint32_t, v);
}

template <int ELEM, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1) k_mx_gemm_exact(MxGemmArgs p) {
    using G = MxGeo<ELEM>;
    __shared__ __attribute__((aligned(16))) uint8_t ring0[G::SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[G::SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[G::SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[G::SLOT];
    __shared__ int rref[2 * kMxTile];  // largest scale byte of each tile row: A rows, then B rows
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int64_t m0 = (int64_t)blockIdx.y * kMxTile, n0 = (int64_t)blockIdx.x * kMxTile;
    const int64_t kb = ELEM == kMxE4M3 ? K : K / 2, ks = K / 32;

    MxSrc<ELEM> src;
    src.ac = p.ac + m0 * kb;
    src.bc = p.bc + n0 * kb;
    src.as = p.as + m0 * ks;
    src.bs = p.bs + n0 * ks;
#pragma unroll
    for (int t = 0; t < G::LOADS; ++t) {
        const int r = 64 * w + G::RPL * t + lane / G::CPR;
        const int c = mx_chunk<G::CPR>(r, lane % G::CPR);
        src.a[t] = (uint32_t)((min(m0 + r, M - 1) - m0) * kb + 16 * c);
        src.b[t] = (uint32_t)((min(n0 + r, N - 1) - n0) * kb + 16 * c);
    }
    src.sa = (uint32_t)((min(m0 + 64 * w + lane, M - 1) - m0) * ks);
    src.sb = (uint32_t)((min(n0 + 64 * w + lane, N - 1) - n0) * ks);

    // each thread: the largest scale byte of one A row and one B row of the
    // tile (rows past the end: the clamped row, never stored)
    rref[tid] = row_max_byte(p.as + min(m0 + tid, M - 1) * ks, ks);
    rref[kMxTile + tid] = row_max_byte(p.bs + min(n0 + tid, N - 1) * ks, ks);

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
        const int64_t pad = (4 - nsteps % 4) % 4, nj = nsteps + pad, last = nsteps - 1;
        auto kc_of = [&](int64_t j) {
            const int64_t kc = j - pad;
            return kc < 0 ? (int64_t)0 : (kc > last ? last : kc);
        };
        if (pad > 0) mx_zero_slot<ELEM>(ring0); else mx_ring_load<ELEM>(src, kc_of(0), ring0, w);
        if (pad > 1) mx_zero_slot<ELEM>(ring1); else mx_ring_load<ELEM>(src, kc_of(1), ring1, w);
        if (pad > 2) mx_zero_slot<ELEM>(ring2); else mx_ring_load<ELEM>(src, kc_of(2), ring2, w);
        mx_ring_load<ELEM>(src, kc_of(3), ring3, w);
        __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(3 * G::LPS));
        __builtin_amdgcn_s_waitcnt(mx_lgkmcnt_zero());
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();  // (also publishes rref)
        asm volatile("" ::: "memory");

        int refa[4], refb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            refa[i] = rref[arow0 + 32 * i + l32];
            refb[i] = rref[kMxTile + brow0 + 32 * i + l32];
        }
        const MxLaneOffsets lo = mx_lane_offsets<ELEM>(arow0, brow0, l32, h);
        // Raw fragments are held once and converted one substep ahead: the
        // MFMAs of substep q alternate with the conversion of substep q + 1
        // (two pairs per MFMA, into the other half of `op`); substep 3 reads
        // the next step's raw fragments (one per MFMA, after their last use
        // in substep 2) and then converts that step's substep 0 (four pairs
        // per MFMA).  sched_barrier keeps the order.
        MxFrags f;
        uint32_t op[2][8][4];  // converted BF16 pairs: A0..A3, B0..B3
        auto scale_of = [&](const MxFrags& fr, int o, int q) {
            const int sh = ELEM == kMxE4M3 ? 8 * (q >> 1) : 0;
            return o < 4 ? pow2_rel((fr.sa[o] >> sh) & 0xFF, refa[o]) : pow2_rel((fr.sb[o - 4] >> sh) & 0xFF, refb[o - 4]);
        };
        auto pair_of = [&](const MxFrags& fr, int o, int q, int pr, float sc) {
            return exact_pair<ELEM>(o < 4 ? fr.a[o] : fr.b[o - 4], q, pr, sc);
        };
#pragma unroll
        for (int o = 0; o < 8; ++o) mx_read_frag_exact<ELEM>(ring0, lo, o, f);
#pragma unroll
        for (int o = 0; o < 8; ++o) {
            const float sc = scale_of(f, o, 0);
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) op[0][o][pr] = pair_of(f, o, 0, pr, sc);
        }

        auto step = [&](int64_t j, uint8_t* cur, uint8_t* nxt) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ob = q & 1;
                if (q == 2) {
                    // half way through the step: own loads of step j + 1
                    // landed, the barrier, then the loads of step j + 4 into
                    // the slot every wave has finished reading
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(2 * G::LPS));
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    mx_ring_load<ELEM>(src, kc_of(j + 4), cur, w);
                    __builtin_amdgcn_sched_barrier(0);
                }
                float sc[8];
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int i = m >> 2, jj = m & 3;
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(v8bf_t, op[ob][i]), __builtin_bit_cast(v8bf_t, op[ob][4 + jj]), acc[i][jj],
                        0, 0, 0);
                    if (q < 3) {
                        // substep q + 1 of this step: two pairs per MFMA
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int pc = 2 * m + u, o = pc >> 2, pr = pc & 3;
                            if (pr == 0) sc[o] = scale_of(f, o, q + 1);
                            op[ob ^ 1][o][pr] = pair_of(f, o, q + 1, pr, sc[o]);
                        }
                    } else if (m < 8) {
                        // the next step's raw fragment m
                        mx_read_frag_exact<ELEM>(nxt, lo, m, f);
                    } else {
                        // the next step's substep 0: four pairs per MFMA
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int pc = 4 * (m - 8) + u, o = pc >> 2, pr = pc & 3;
                            if (pr == 0) sc[o] = scale_of(f, o, 0);
                            op[ob ^ 1][o][pr] = pair_of(f, o, 0, pr, sc[o]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        for (int64_t j = 0; j < nj; j += 4) {
            step(j, ring0, ring1);
            step(j + 1, ring1, ring2);
            step(j + 2, ring2, ring3);
            step(j + 3, ring3, ring0);
        }
        __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(0));
    } else {
        __syncthreads();  // (K == 0: rref published for the epilogue)
    }

    // C = 2^(R_A[m] + R_B[n] - 254) * acc (exact unless C leaves binary32's
    // normal range); accumulator r of tile (i, j): row 32 i + 8 (r / 4) + 4 h +
    // r % 4, column 32 j + l32 of the wave tile
    const int64_t nw = n0 + brow0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = nw + 32 * j + l32;
            if (c >= N) continue;
            const int rb = rref[kMxTile + brow0 + 32 * j + l32];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = arow0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                const int64_t m = m0 + rl;
                if (m < M) {
                    const float v = ldexpf(acc[i][j][r], rref[rl] + rb - 254);
                    if (OUT_BF16)
                        static_cast<uint16_t*>(p.C)[m * p.ldc + c] = (uint16_t)__builtin_bit_cast(uint16_t, (__bf16)v);
                    else
                        static_cast<float*>(p.C)[m * p.ldc + c] = v;
                }
            }
        }
}

// ============================================================ full-line kernel
// For K % 1024 == 0 with 16-byte-aligned scale rows (every benchmarked shape):
// the ring kernel's 256 x 256 tile with the memory traffic shaped for gfx950's
// caches, where each distinct cache line a wave-wide load touches costs
// about the same whatever part of it is used, and eight waves:
//   - a slot holds 128 bytes of every tile row (a whole line): 2 K steps of
//     E4M3 or 4 of E2M1 ("a chunk"); two slots, the next chunk's loads in
//     flight while the current chunk is consumed; a chunk's last step opens
//     with the wait and barrier that hand its slot to the loads of the chunk
//     after next;
//   - scale bytes arrive 16 per row (8 K steps) per load, one group ahead,
//     into two small buffers;
//   - 16-byte chunk c of slot row r sits at chunk c ^ (r % 8) ^ ((r / 8) % 4)
//     (bits 0..4 of r), which spreads the fragment reads over every bank for
//     8 lanes (32 banks) and for 16 lanes (64 banks);
//   - eight waves, two per SIMD, in a 2 x 4 grid of 128 x 64 wave tiles (4 x 2
//     MFMA tiles, 128 accumulators per lane): while one wave of a SIMD waits
//     for its LDS reads or at the barrier the other issues MFMAs.  Against
//     four waves of 128 x 128 (one per SIMD, fragments double-buffered),
//     8192^3 ran 0.552 -> 0.464 ms with E4M3 and 0.307 -> 0.287 ms with E2M1,
//     20480 x 5120 x 8192 0.939 -> 0.788 and 0.534 -> 0.494 ms, outputs bit
//     for bit the same (alternating A/B on one box).
// The body is unrolled over 16 K steps (8 E4M3 or 4 E2M1 chunks, 2 scale
// groups), so every slot and buffer has a static name and there is no
// padding.
template <int ELEM>
struct MxFull {
    static constexpr int SPC = ELEM == kMxE4M3 ? 2 : 4;  // K steps per chunk
    static constexpr int CODES = kMxTile * 128;          // code bytes per operand per slot
    static constexpr int SCB = kMxTile * 16;             // scale bytes per operand per group buffer
    static constexpr int FMT = ELEM == kMxE4M3 ? 0 : 4;
};

// (row bits 0..4 only: fragment rows 32 apart share it)
__device__ __forceinline__ int mx_full_swz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// Per-lane byte offsets of the ring loads: code row r of load t in chunk 0
// (add 128 per chunk), scale row (add 16 per group).
struct MxFullSrc {
    const uint8_t *ac, *bc, *as, *bs;
    uint32_t a[8], b[8];
    uint32_t sa, sb;
};

// Fragments are held once (no second register set): the next step's fragment
// of an A tile is read right after the step's last MFMA on that tile, a B
// fragment after its last MFMA, with the MFMAs ordered B tile by B tile so
// that each read has at least three MFMAs of the step after to land.  Each
// wave loads 32 rows of each operand per chunk and, per scale group, the 16
// scale bytes of 32 A rows (lanes 0..31) and of 32 B rows (lanes 32..63):
// wave w's 1 KiB of a group buffer holds A rows 32 w .. 32 w + 31, then B rows
// 32 w .. 32 w + 31.
// (each 32-bit lane offset passes through an empty asm statement at the load:
// the compiler then cannot hoist the 64-bit per-lane addresses out of the
// loop, where they would hold two registers each, and forms the address as a
// scalar base plus the offset)
template <int ELEM>
__device__ __forceinline__ void mx_full8_chunk_load(const MxFullSrc& src, int64_t chunk, uint8_t* slot, int w) {
    using F = MxFull<ELEM>;
    const uint8_t* ac = src.ac + chunk * 128;
    const uint8_t* bc = src.bc + chunk * 128;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t o = src.a[t];
        asm volatile("" : "+v"(o));
        __builtin_amdgcn_global_load_lds((gmem_t*)(ac + o), (lmem_t*)(slot + (32 * w + 8 * t) * 128), 16, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t o = src.b[t];
        asm volatile("" : "+v"(o));
        __builtin_amdgcn_global_load_lds((gmem_t*)(bc + o), (lmem_t*)(slot + F::CODES + (32 * w + 8 * t) * 128), 16,
                                         0, 0);
    }
}

// (one load: each lane's address picks A (lanes 0..31) or B (lanes 32..63))
__device__ __forceinline__ void mx_full8_scale_load(const uint8_t* as, const uint8_t* bs, uint32_t so, int lane,
                                                    int64_t group, uint8_t* buf, int w) {
    const uint8_t* sp = (lane < 32 ? as : bs) + group * 16 + so;
    __builtin_amdgcn_global_load_lds((gmem_t*)sp, (lmem_t*)(buf + 1024 * w), 16, 0, 0);
}

// A lane's LDS byte offsets for the 8-wave kernel: code piece q of a fragment
// row inside a slot (E4M3: q = 2 t + hi, t the step of the chunk, hi the upper
// 16 bytes; E2M1: q = t) for A (tile 0 of the wave; tile i adds 4096 i) and
// for B, and its scale byte inside a group buffer (A tile 0 / B tile 0, step
// 0; tile i adds 1024 i, step g adds 2 g).  They are formed once and made
// opaque to the compiler, so that every fragment read is one of them plus an
// immediate instead of a register of its own per tile, step and slot.
struct MxFull8Offsets {
    uint32_t a[4], b[4];
    uint32_t sa, sb;
};

template <int ELEM>
__device__ __forceinline__ MxFull8Offsets mx_full8_offsets(int wm, int wn, int l32, int h) {
    using F = MxFull<ELEM>;
    MxFull8Offsets o;
    const int sw = mx_full_swz(l32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = ELEM == kMxE4M3 ? (4 * (q >> 1) + 2 * (q & 1) + h) : (2 * q + h);
        o.a[q] = (uint32_t)((128 * wm + l32) * 128 + 16 * (c ^ sw));
        o.b[q] = (uint32_t)(F::CODES + (64 * wn + l32) * 128 + 16 * (c ^ sw));
        asm volatile("" : "+v"(o.a[q]));
        asm volatile("" : "+v"(o.b[q]));
    }
    o.sa = (uint32_t)(1024 * (4 * wm) + 16 * l32 + h);
    o.sb = (uint32_t)(1024 * (2 * wn) + 512 + 16 * l32 + h);
    asm volatile("" : "+v"(o.sa));
    asm volatile("" : "+v"(o.sb));
    return o;
}

// Fragment f of the next step (f = 0..3: A tile f, 4..5: B tile f - 4) from
// step t of the slot, with its scale byte (step g of the group buffer).
template <int ELEM>
__device__ __forceinline__ void mx_full8_read(const uint8_t* slot, const uint8_t* sbuf, int t, int g, int f,
                                              const MxFull8Offsets& o, v8i_t (&a)[4], v8i_t (&b)[2], int (&sa)[4],
                                              int (&sb)[2]) {
    const bool isb = f >= 4;
    const int i = isb ? f - 4 : f;
    v8i_t v;
    if constexpr (ELEM == kMxE4M3) {
        const uint32_t lo = isb ? o.b[2 * t] : o.a[2 * t], hi = isb ? o.b[2 * t + 1] : o.a[2 * t + 1];
        const v4i_t ql = lds16(slot + lo + 4096 * i), qh = lds16(slot + hi + 4096 * i);
        v = v8i_t{ql[0], ql[1], ql[2], ql[3], qh[0], qh[1], qh[2], qh[3]};
    } else {
        const uint32_t off = isb ? o.b[t] : o.a[t];
        const v4i_t q = lds16(slot + off + 4096 * i);
        v = v8i_t{q[0], q[1], q[2], q[3], 0, 0, 0, 0};
    }
    const int sbyte = sbuf[(isb ? o.sb : o.sa) + 1024 * i + 2 * g];
    if (isb) {
        b[i] = v;
        sb[i] = sbyte;
    } else {
        a[i] = v;
        sa[i] = sbyte;
    }
}

// Logical tile lg -> tile (row-major index): logical tiles run down each
// group of 4 tile rows column by column, so that consecutive logical tiles
// (the ones an XCD runs at once) share A rows and B rows, also where the
// grid is narrow (a 20-tile row would otherwise spread one XCD's 32 tiles
// over 13 tile rows and 5 columns instead of 4 x 8).  A bijection on the
// grid's tiles; the last group may hold fewer rows.
__device__ __forceinline__ int mx_tile_of(const MxGemmArgs& p, int lg) {
    const int rows = (int)((p.M + kMxTile - 1) / kMxTile), gsz = 4 * p.tiles_x;
    const int grp = lg / gsz, first = 4 * grp, gm = min(rows - first, 4), r = lg - grp * gsz;
    return (first + r % gm) * p.tiles_x + r / gm;
}

// Work item L = first + bx of a full-line workgroup bx: tile L whole
// (L < t_main), or part s of tile t_main + j / split (j = L - t_main,
// s = j % split), which takes units [s U / split, (s + 1) U / split) of the
// U units of 16 K steps.
struct MxWork {
    int tile, part, u0, u1;
};
__device__ __forceinline__ MxWork mx_work(const MxGemmArgs& p, int units, uint32_t bx) {
    MxWork w{p.first + (int)bx, -1, 0, units};
    if (w.tile >= p.t_main) {
        const int j = w.tile - p.t_main, sp = j % p.split;
        w.tile = p.t_main + j / p.split;
        w.part = j;
        w.u0 = sp * units / p.split;
        w.u1 = (sp + 1) * units / p.split;
    } else {
        // workgroups are dealt to the 8 XCDs in turn (L to XCD L % 8): of the
        // first t8 (t_main rounded down to a multiple of 8), XCD x's take the
        // x-th eighth of those logical tiles in order
        const int t8 = p.t_main & ~7;
        if (w.tile < t8) w.tile = (w.tile & 7) * (t8 >> 3) + (w.tile >> 3);
    }
    w.tile = mx_tile_of(p, w.tile);
    return w;
}

template <int ELEM, bool OUT_BF16>
__global__ void __launch_bounds__(512, 1) k_mx_gemm_full8(MxGemmArgs p) {
    using F = MxFull<ELEM>;
    constexpr int SPC = F::SPC;
    __shared__ __attribute__((aligned(16))) uint8_t slot0[2 * F::CODES];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[2 * F::CODES];
    __shared__ __attribute__((aligned(16))) uint8_t scb0[2 * F::SCB];
    __shared__ __attribute__((aligned(16))) uint8_t scb1[2 * F::SCB];
    static_assert(2 * F::SCB == 8 * 1024, "scale group buffer: 1 KiB per wave");
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6) & 7;
    const int wm = w >> 2, wn = w & 3;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t M = p.M, N = p.N, K = p.K;
    // (32-bit step, chunk and group counts: K < 2^31)
    const int units = (int)(K / 1024);  // units of 16 K steps
    const MxWork wk = mx_work(p, units, blockIdx.x);  // uniform across the workgroup
    const int u0 = wk.u0, u1 = wk.u1;
    __builtin_assume(u1 > u0);  // every work item has at least one unit (split <= units)
    const int64_t m0 = (int64_t)(wk.tile / p.tiles_x) * kMxTile, n0 = (int64_t)(wk.tile % p.tiles_x) * kMxTile;
    const int64_t kb = ELEM == kMxE4M3 ? K : K / 2, ks = K / 32;

    MxFullSrc src;
    src.ac = p.ac + m0 * kb;
    src.bc = p.bc + n0 * kb;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int r = 32 * w + 8 * t + (lane >> 3);
        const int c = (lane & 7) ^ mx_full_swz(r);  // the swizzle is an involution
        src.a[t] = (uint32_t)((min(m0 + r, M - 1) - m0) * kb + 16 * c);
        src.b[t] = (uint32_t)((min(n0 + r, N - 1) - n0) * kb + 16 * c);
    }
    // this lane's scale row: A row 32 w + lane (lanes 0..31), B row 32 w + lane - 32,
    // as an offset from the tile's first row
    const uint8_t* s_as = p.as + m0 * ks;
    const uint8_t* s_bs = p.bs + n0 * ks;
    const uint32_t so = (uint32_t)(lane < 32 ? (min(m0 + 32 * w + lane, M - 1) - m0) * ks
                                             : (min(n0 + 32 * w + (lane - 32), N - 1) - n0) * ks);

    v16f_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const MxFull8Offsets off = mx_full8_offsets<ELEM>(wm, wn, l32, h);
    // the range's chunks and scale groups (a unit is an even number of
    // chunks and two groups, so its first chunk and group go to slot 0 and
    // buffer 0, as the loop expects)
    const int c_end = 16 * u1 / SPC, g_end = 2 * u1, c_first = 16 * u0 / SPC, g_first = 2 * u0;
    auto cclamp = [&](int c) { return c < c_end ? c : c_end - 1; };
    auto gclamp = [&](int g) { return g < g_end ? g : g_end - 1; };

    // prologue: the range's first two scale groups and chunks (a unit holds both)
    mx_full8_scale_load(s_as, s_bs, so, lane, g_first, scb0, w);
    mx_full8_scale_load(s_as, s_bs, so, lane, g_first + 1, scb1, w);
    mx_full8_chunk_load<ELEM>(src, c_first, slot0, w);
    mx_full8_chunk_load<ELEM>(src, c_first + 1, slot1, w);
    __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(8));  // all but chunk 1
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    v8i_t fa[4], fb[2];
    int sa[4], sb[2];
#pragma unroll
    for (int f = 0; f < 6; ++f) mx_full8_read<ELEM>(slot0, scb0, 0, 0, f, off, fa, fb, sa, sb);

    for (int it = 16 * u0; it < 16 * u1; it += 16) {
        const int chunk0 = it / SPC, group0 = it / 8;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int cc = s / SPC, t = s % SPC, g = s % 8;
            uint8_t* slot = (cc & 1) ? slot1 : slot0;
            uint8_t* other = (cc & 1) ? slot0 : slot1;
            uint8_t* gbuf = (s / 8) ? scb1 : scb0;  // this step's scale group
            // where the next step's fragments and scale bytes are
            const uint8_t* nslot = (t == SPC - 1) ? other : slot;
            const int nt = (t == SPC - 1) ? 0 : t + 1;
            const uint8_t* nsbuf = (g == 7) ? ((s == 7) ? scb1 : scb0) : gbuf;
            const int ng = (g == 7) ? 0 : g + 1;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                if (m == 0) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (t == SPC - 1) {
                        // the next chunk's loads (and any scale group issued
                        // before them) landed and this step's fragments are in
                        // registers; after the barrier every wave has read all
                        // of this chunk's slot
                        __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(0) & mx_lgkmcnt_zero());
                        asm volatile("" ::: "memory");
                        __builtin_amdgcn_s_barrier();
                        asm volatile("" ::: "memory");
                        if (g == 7) mx_full8_scale_load(s_as, s_bs, so, lane, gclamp(group0 + s / 8 + 2), gbuf, w);
                        mx_full8_chunk_load<ELEM>(src, cclamp(chunk0 + cc + 2), slot, w);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int i = m & 3, j = m >> 2;
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fa[i], fb[j], acc[i][j], F::FMT, F::FMT, 0, sa[i], 0, sb[j]);
                // next step: B tile 0 after its last MFMA (m = 3), A tile i
                // after its last (m = 4 + i), B tile 1 after m = 7
                if (m == 3) mx_full8_read<ELEM>(nslot, nsbuf, nt, ng, 4, off, fa, fb, sa, sb);
                if (m >= 4) mx_full8_read<ELEM>(nslot, nsbuf, nt, ng, m - 4, off, fa, fb, sa, sb);
                if (m == 7) mx_full8_read<ELEM>(nslot, nsbuf, nt, ng, 5, off, fa, fb, sa, sb);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(0));

    // output: C, or (a part of a split tile; FP32 instances only) the part's
    // 256 x 256 matrix, through the same code.  The work item is found again
    // from an opaque copy of the workgroup index rather than kept through
    // the loop (kept, the tile's origin cost registers the loop needs).
    // (the divisors made opaque too: otherwise their reciprocals, shared
    // with the first computation, are what is kept)
    uint32_t bx = blockIdx.x;
    MxGemmArgs pe = p;
    asm volatile("" : "+s"(bx), "+s"(pe.tiles_x), "+s"(pe.split), "+s"(pe.t_main), "+s"(pe.first));
    const MxWork we = mx_work(pe, units, bx);
    void* Cp = p.C;
    int64_t ldcp = p.ldc, Me = M, Ne = N;
    int64_t mt = (int64_t)(we.tile / pe.tiles_x) * kMxTile, nt0 = (int64_t)(we.tile % pe.tiles_x) * kMxTile;
    if constexpr (!OUT_BF16) {
        if (we.part >= 0) {
            Cp = p.parts + (int64_t)we.part * kMxTile * kMxTile;
            ldcp = kMxTile;
            Me = Ne = kMxTile;
            mt = nt0 = 0;
        }
    }
    const int64_t mw = mt + 128 * wm, nw = nt0 + 64 * wn;
    if (mw + 128 <= Me && nw + 64 <= Ne &&
        store_wave_block<4, 2, OUT_BF16>(Cp, ldcp, mw, nw, h, l32,
                                         [&](int i, int j, int r) { return acc[i][j][r]; }))
        return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t c = nw + 32 * j + l32;
            if (c >= Ne) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = mw + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < Me) {
                    if (OUT_BF16)
                        static_cast<uint16_t*>(Cp)[m * ldcp + c] =
                            (uint16_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][r]);
                    else
                        static_cast<float*>(Cp)[m * ldcp + c] = acc[i][j][r];
                }
            }
        }
}

// The tail tiles of a split full-line launch: element (r, c) of tile
// t_main + blockIdx.x is the sum of its parts' element (r, c), added in part
// order (deterministic), rounded to BF16 as the epilogues round for BF16
// outputs.  Workgroup (x, y) covers 16 rows from
// 16 y of the tile.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) k_mx_tail_sum(MxGemmArgs p) {
    const int tile = mx_tile_of(p, p.t_main + (int)blockIdx.x);
    const int64_t m0 = (int64_t)(tile / p.tiles_x) * kMxTile, n0 = (int64_t)(tile % p.tiles_x) * kMxTile;
    const float* part0 = p.parts + (int64_t)blockIdx.x * p.split * kMxTile * kMxTile;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 4 * (256 * k + threadIdx.x);  // first of 4 elements in 16 rows x 256
        const int r = 16 * blockIdx.y + e / kMxTile, c = e % kMxTile;
        float4 v = *reinterpret_cast<const float4*>(part0 + r * kMxTile + c);
        for (int s = 1; s < p.split; ++s) {
            const float4 u =
                *reinterpret_cast<const float4*>(part0 + (int64_t)s * kMxTile * kMxTile + r * kMxTile + c);
            v.x += u.x;
            v.y += u.y;
            v.z += u.z;
            v.w += u.w;
        }
        const int64_t m = m0 + r;
        if (m >= p.M) continue;
        const float o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + c + q;
            if (n >= p.N) break;
            if (OUT_BF16)
                static_cast<uint16_t*>(p.C)[m * p.ldc + n] = (uint16_t)__builtin_bit_cast(uint16_t, (__bf16)o[q]);
            else
                static_cast<float*>(p.C)[m * p.ldc + n] = o[q];
        }
    }
}

// ============================================================ full-line exact kernel
// Exact accumulation (as k_mx_gemm_exact) for K % 1024 == 0 with 16-byte-
// aligned scale rows: the full-line kernel's slots (128 bytes of every tile
// row per chunk, two slots) and scale groups (16 bytes per row, two buffers),
// one barrier per chunk instead of one per K step, with four waves of
// 128 x 128 tiles and the exact kernel's substep schedule: raw fragments held
// once, substep q + 1 converted between the MFMAs of substep q, the next
// step's raw fragments read in substep 3 (after a chunk's last step has passed
// the barrier that hands the other slot over) and its substep 0 converted in
// the second half of substep 3.  Each wave loads 64 rows of each operand per
// chunk and their 16 scale bytes per group.
template <int ELEM>
__device__ __forceinline__ void mx_full4_chunk_load(const MxFullSrc& src, int64_t chunk, uint8_t* slot, int w) {
    using F = MxFull<ELEM>;
    const uint8_t* ac = src.ac + chunk * 128;
    const uint8_t* bc = src.bc + chunk * 128;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t o = src.a[t];
        asm volatile("" : "+v"(o));
        __builtin_amdgcn_global_load_lds((gmem_t*)(ac + o), (lmem_t*)(slot + (64 * w + 8 * t) * 128), 16, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t o = src.b[t];
        asm volatile("" : "+v"(o));
        __builtin_amdgcn_global_load_lds((gmem_t*)(bc + o), (lmem_t*)(slot + F::CODES + (64 * w + 8 * t) * 128), 16,
                                         0, 0);
    }
}
constexpr int kMxFull4ChunkLoads = 16;

template <int ELEM>
__device__ __forceinline__ void mx_full4_scale_load(const MxFullSrc& src, int64_t group, uint8_t* buf, int w) {
    using F = MxFull<ELEM>;
    uint32_t oa = src.sa, ob = src.sb;
    asm volatile("" : "+v"(oa));
    asm volatile("" : "+v"(ob));
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.as + group * 16 + oa), (lmem_t*)(buf + 64 * w * 16), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.bs + group * 16 + ob), (lmem_t*)(buf + F::SCB + 64 * w * 16), 16, 0,
                                     0);
}

// A lane's LDS byte offsets for the exact full-line kernel: code piece q of
// its A tile 0 / B tile 0 row (E4M3: q = 2 t + hi; E2M1: q = t; tile i adds
// 4096 i) and the rows' 16 scale bytes (tile i adds 512 i), opaque to the
// compiler so that each read is one of them plus an immediate.
struct MxExact4Offsets {
    uint32_t a[4], b[4];
    uint32_t sa, sb;
};

template <int ELEM>
__device__ __forceinline__ MxExact4Offsets mx_exact4_offsets(int wm, int wn, int l32, int h) {
    using F = MxFull<ELEM>;
    MxExact4Offsets o;
    const int sw = mx_full_swz(l32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = ELEM == kMxE4M3 ? (4 * (q >> 1) + 2 * (q & 1) + h) : (2 * q + h);
        o.a[q] = (uint32_t)((128 * wm + l32) * 128 + 16 * (c ^ sw));
        o.b[q] = (uint32_t)(F::CODES + (128 * wn + l32) * 128 + 16 * (c ^ sw));
        asm volatile("" : "+v"(o.a[q]));
        asm volatile("" : "+v"(o.b[q]));
    }
    o.sa = (uint32_t)((128 * wm + l32) * 16);
    o.sb = (uint32_t)(F::SCB + (128 * wn + l32) * 16);
    asm volatile("" : "+v"(o.sa));
    asm volatile("" : "+v"(o.sb));
    return o;
}

// Raw fragment o (0..3: A tile o, 4..7: B tile o - 4) of step t of a chunk,
// with the scale bytes its conversion needs from step g of the group buffer
// (E4M3: both blocks of the step, block 0 in bits 0..7; E2M1: block h).
template <int ELEM>
__device__ __forceinline__ void mx_exact4_read(const uint8_t* slot, const uint8_t* sbuf, int t, int g, int o, int h,
                                               const MxExact4Offsets& off, MxFrags& f) {
    const bool isb = o >= 4;
    const int i = isb ? o - 4 : o;
    v8i_t v;
    if constexpr (ELEM == kMxE4M3) {
        const uint32_t lo = isb ? off.b[2 * t] : off.a[2 * t], hi = isb ? off.b[2 * t + 1] : off.a[2 * t + 1];
        const v4i_t ql = lds16(slot + lo + 4096 * i), qh = lds16(slot + hi + 4096 * i);
        v = v8i_t{ql[0], ql[1], ql[2], ql[3], qh[0], qh[1], qh[2], qh[3]};
    } else {
        const v4i_t q = lds16(slot + (isb ? off.b[t] : off.a[t]) + 4096 * i);
        v = v8i_t{q[0], q[1], q[2], q[3], 0, 0, 0, 0};
    }
    const uint8_t* sp = sbuf + (isb ? off.sb : off.sa) + 512 * i + 2 * g;
    int sc;
    if constexpr (ELEM == kMxE4M3) sc = *reinterpret_cast<const uint16_t*>(sp);
    else sc = sp[h];
    if (isb) {
        f.b[i] = v;
        f.sb[i] = sc;
    } else {
        f.a[i] = v;
        f.sa[i] = sc;
    }
}

template <int ELEM, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1) k_mx_gemm_exact_full(MxGemmArgs p) {
    using F = MxFull<ELEM>;
    constexpr int SPC = F::SPC;
    __shared__ __attribute__((aligned(16))) uint8_t slot0[2 * F::CODES];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[2 * F::CODES];
    __shared__ __attribute__((aligned(16))) uint8_t scb0[2 * F::SCB];
    __shared__ __attribute__((aligned(16))) uint8_t scb1[2 * F::SCB];
    __shared__ int rref[2 * kMxTile];  // largest scale byte of each tile row: A rows, then B rows
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int units = (int)(K / 1024);  // units of 16 K steps
    const MxWork wk = mx_work(p, units, blockIdx.x);  // uniform across the workgroup
    const int u0 = wk.u0, u1 = wk.u1;
    const int64_t m0 = (int64_t)(wk.tile / p.tiles_x) * kMxTile, n0 = (int64_t)(wk.tile % p.tiles_x) * kMxTile;
    const int64_t kb = ELEM == kMxE4M3 ? K : K / 2, ks = K / 32;

    MxFullSrc src;
    src.ac = p.ac + m0 * kb;
    src.bc = p.bc + n0 * kb;
    src.as = p.as + m0 * ks;
    src.bs = p.bs + n0 * ks;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int r = 64 * w + 8 * t + (lane >> 3);
        const int c = (lane & 7) ^ mx_full_swz(r);  // the swizzle is an involution
        src.a[t] = (uint32_t)((min(m0 + r, M - 1) - m0) * kb + 16 * c);
        src.b[t] = (uint32_t)((min(n0 + r, N - 1) - n0) * kb + 16 * c);
    }
    src.sa = (uint32_t)((min(m0 + 64 * w + lane, M - 1) - m0) * ks);
    src.sb = (uint32_t)((min(n0 + 64 * w + lane, N - 1) - n0) * ks);

    // each thread: the largest scale byte of one A row and one B row of the
    // tile (rows past the end: the clamped row, never stored)
    rref[tid] = row_max_byte(p.as + min(m0 + tid, M - 1) * ks, ks);
    rref[kMxTile + tid] = row_max_byte(p.bs + min(n0 + tid, N - 1) * ks, ks);

    v16f_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const MxExact4Offsets off = mx_exact4_offsets<ELEM>(wm, wn, l32, h);
    // the range's chunks and scale groups (a unit is an even number of
    // chunks and two groups: its first chunk and group go to slot 0, buffer 0)
    const int c_end = 16 * u1 / SPC, g_end = 2 * u1, c_first = 16 * u0 / SPC, g_first = 2 * u0;
    auto cclamp = [&](int c) { return c < c_end ? c : c_end - 1; };
    auto gclamp = [&](int g) { return g < g_end ? g : g_end - 1; };

    // prologue: the range's first two scale groups and chunks (a unit holds both)
    mx_full4_scale_load<ELEM>(src, g_first, scb0, w);
    mx_full4_scale_load<ELEM>(src, g_first + 1, scb1, w);
    mx_full4_chunk_load<ELEM>(src, c_first, slot0, w);
    mx_full4_chunk_load<ELEM>(src, c_first + 1, slot1, w);
    __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(kMxFull4ChunkLoads));  // all but chunk 1
    __builtin_amdgcn_s_waitcnt(mx_lgkmcnt_zero());
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();  // (also publishes rref)
    asm volatile("" ::: "memory");

    int refa[4], refb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        refa[i] = rref[128 * wm + 32 * i + l32];
        refb[i] = rref[kMxTile + 128 * wn + 32 * i + l32];
    }
    MxFrags f;
    uint32_t op[2][8][4];  // converted BF16 pairs: A0..A3, B0..B3
    auto scale_of = [&](int o, int q) {
        const int sh = ELEM == kMxE4M3 ? 8 * (q >> 1) : 0;
        return o < 4 ? pow2_rel((f.sa[o] >> sh) & 0xFF, refa[o]) : pow2_rel((f.sb[o - 4] >> sh) & 0xFF, refb[o - 4]);
    };
    auto pair_of = [&](int o, int q, int pr, float sc) {
        return exact_pair<ELEM>(o < 4 ? f.a[o] : f.b[o - 4], q, pr, sc);
    };
#pragma unroll
    for (int o = 0; o < 8; ++o) mx_exact4_read<ELEM>(slot0, scb0, 0, 0, o, h, off, f);
#pragma unroll
    for (int o = 0; o < 8; ++o) {
        const float sc = scale_of(o, 0);
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) op[0][o][pr] = pair_of(o, 0, pr, sc);
    }

    for (int it = 16 * u0; it < 16 * u1; it += 16) {
        const int chunk0 = it / SPC, group0 = it / 8;
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int cc = s / SPC, t = s % SPC, g = s % 8;
            uint8_t* slot = (cc & 1) ? slot1 : slot0;
            uint8_t* other = (cc & 1) ? slot0 : slot1;
            uint8_t* gbuf = (s / 8) ? scb1 : scb0;  // this step's scale group
            // where the next step's fragments and scale bytes are
            const uint8_t* nslot = (t == SPC - 1) ? other : slot;
            const int nt = (t == SPC - 1) ? 0 : t + 1;
            const uint8_t* nsbuf = (g == 7) ? ((s == 7) ? scb1 : scb0) : gbuf;
            const int ng = (g == 7) ? 0 : g + 1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int ob = q & 1;
                float sc[8];
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    if (q == 3 && m == 0 && t == SPC - 1) {
                        // the next chunk's loads (and any scale group issued
                        // before them) landed, this step's fragments are in
                        // registers; after the barrier every wave has read all
                        // of this chunk's slot, which takes the chunk after next
                        __builtin_amdgcn_sched_barrier(0);
                        __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(0) & mx_lgkmcnt_zero());
                        asm volatile("" ::: "memory");
                        __builtin_amdgcn_s_barrier();
                        asm volatile("" ::: "memory");
                        if (g == 7) mx_full4_scale_load<ELEM>(src, gclamp(group0 + s / 8 + 2), gbuf, w);
                        mx_full4_chunk_load<ELEM>(src, cclamp(chunk0 + cc + 2), slot, w);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    const int i = m >> 2, jj = m & 3;
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(v8bf_t, op[ob][i]), __builtin_bit_cast(v8bf_t, op[ob][4 + jj]), acc[i][jj],
                        0, 0, 0);
                    if (q < 3) {
                        // substep q + 1 of this step: two pairs per MFMA
#pragma unroll
                        for (int u = 0; u < 2; ++u) {
                            const int pc = 2 * m + u, o = pc >> 2, pr = pc & 3;
                            if (pr == 0) sc[o] = scale_of(o, q + 1);
                            op[ob ^ 1][o][pr] = pair_of(o, q + 1, pr, sc[o]);
                        }
                    } else if (m < 8) {
                        // the next step's raw fragment m
                        mx_exact4_read<ELEM>(nslot, nsbuf, nt, ng, m, h, off, f);
                    } else {
                        // the next step's substep 0: four pairs per MFMA
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int pc = 4 * (m - 8) + u, o = pc >> 2, pr = pc & 3;
                            if (pr == 0) sc[o] = scale_of(o, 0);
                            op[ob ^ 1][o][pr] = pair_of(o, 0, pr, sc[o]);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
    // the last look-ahead loads (clamped re-reads) land before the LDS is released
    __builtin_amdgcn_s_waitcnt(mx_vmcnt_at_most(0));

    // output: C, or (a part of a split tile; FP32 instances only) the part's
    // 256 x 256 matrix of scaled sums, through the same code; the work item
    // found again from opaque copies (as in k_mx_gemm_full8)
    uint32_t bx = blockIdx.x;
    MxGemmArgs pe = p;
    asm volatile("" : "+s"(bx), "+s"(pe.tiles_x), "+s"(pe.split), "+s"(pe.t_main), "+s"(pe.first));
    const MxWork we = mx_work(pe, units, bx);
    void* Cp = p.C;
    int64_t ldcp = p.ldc, Me = M, Ne = N;
    int64_t mt = (int64_t)(we.tile / pe.tiles_x) * kMxTile, nt0 = (int64_t)(we.tile % pe.tiles_x) * kMxTile;
    if constexpr (!OUT_BF16) {
        if (we.part >= 0) {
            Cp = p.parts + (int64_t)we.part * kMxTile * kMxTile;
            ldcp = kMxTile;
            Me = Ne = kMxTile;
            mt = nt0 = 0;
        }
    }
    const int64_t nw = nt0 + 128 * wn;
    if (mt + 128 * wm + 128 <= Me && nw + 128 <= Ne &&
        store_wave_block<4, 4, OUT_BF16>(Cp, ldcp, mt + 128 * wm, nw, h, l32, [&](int i, int j, int r) {
            return ldexpf(acc[i][j][r], rref[128 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3)] +
                                            rref[kMxTile + 128 * wn + 32 * j + l32] - 254);
        }))
        return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t c = nw + 32 * j + l32;
            if (c >= Ne) continue;
            const int rb = rref[kMxTile + 128 * wn + 32 * j + l32];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = 128 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                const int64_t m = mt + rl;
                if (m < Me) {
                    const float v = ldexpf(acc[i][j][r], rref[rl] + rb - 254);
                    if (OUT_BF16)
                        static_cast<uint16_t*>(Cp)[m * ldcp + c] = (uint16_t)__builtin_bit_cast(uint16_t, (__bf16)v);
                    else
                        static_cast<float*>(Cp)[m * ldcp + c] = v;
                }
            }
        }
}

inline int64_t mx_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Split of the full-line kernels' last partial round of tiles: as
// gemm_split_plan, in whole units of 1024 K, when it pays (below).
// Time of one tile's 1024 K when its round is the last and runs alone, in µs
// (native E2M1 measured on a single round of 9 tiles at K = 4096; the others
// scaled from it by their measured whole-chip rates).
double mx_split_tile_us(int elem, bool exact) {
    if (exact) return elem == kMxE2M1 ? 20.5 : 23.0;
    return elem == kMxE2M1 ? 7.0 : 11.4;
}

// A split of U units of 1024 K into q parts ends when its longest part,
// ceil(U / q) units, does, so it saves U - ceil(U / q) units of a lone
// tile's time.  It costs about 1.5 µs + 2.6 µs per part (the second launch
// and the sum kernel, whose reads grow with q) plus 0.3 µs per MiB of parts
// written and re-read (fitted to timings of 9- and 64-tile last rounds at
// K = 2048 and 4096).  The plan takes the q with the largest positive gain,
// else no split.
GemmSplit mx_gemm_split_plan(int64_t M, int64_t N, int64_t K, double tile_us, int cus) {
    GemmSplit sp{0, 1, 0};
    if (M <= 0 || N <= 0 || K <= 0 || K % 1024 || cus <= 0) return sp;
    const int64_t tiles = mx_cdiv(N, kMxTile) * mx_cdiv(M, kMxTile), tail = tiles % cus;
    sp.t_main = tiles;
    if (tail == 0) return sp;
    const int64_t smax = std::min<int64_t>(std::min<int64_t>(cus / tail, K / 1024), kMaxTailSplit);
    int64_t split = 1;
    double best = 0.0;
    for (int64_t q = 2; q <= smax; ++q) {
        const int64_t units = K / 1024, longest = (units + q - 1) / q;
        const double gain =
            tile_us * (double)(units - longest) - 1.5 - 2.6 * (double)q - 0.3 * 0.25 * (double)(tail * q);
        if (gain > best) best = gain, split = q;
    }
    if (split < 2) return sp;
    sp.t_main = tiles - tail;
    sp.split = (int)split;
    sp.bytes = tail * split * (int64_t)kMxTile * kMxTile * 4;
    return sp;
}

hipError_t launch_mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int elem, int64_t M, int64_t N, int64_t K, void* C,
                          bool c_bf16, int64_t ldc, bool exact, void* ws, size_t ws_bytes, hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    MxGemmArgs p{a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, 0, 0, 1, nullptr, 0};
    dim3 grid((unsigned)mx_cdiv(N, kMxTile), (unsigned)mx_cdiv(M, kMxTile));
    const bool full = K % 1024 == 0 && K > 0 && (reinterpret_cast<uintptr_t>(a_scales) & 15) == 0 &&
                      (reinterpret_cast<uintptr_t>(b_scales) & 15) == 0;
    // the full-line kernels take a one-dimensional grid of work items: the
    // whole tiles, then the parts of a split last round
    const int64_t tiles = (int64_t)grid.x * grid.y;
    p.tiles_x = (int)grid.x;
    p.t_main = (int)tiles;
    if (full && ws) {
        int cus = 0;
        const hipError_t e = device_cus(cus);
        if (e != hipSuccess) return e;
        const GemmSplit plan = mx_gemm_split_plan(M, N, K, mx_split_tile_us(elem, exact), cus);
        if (plan.split > 1 && (size_t)plan.bytes <= ws_bytes) {
            p.t_main = (int)plan.t_main;
            p.split = plan.split;
            p.parts = static_cast<float*>(ws);
        }
    }
    const int64_t tail = tiles - p.t_main;
    // the parts run in the FP32 instance (their sums are binary32): with a
    // BF16 output, a second launch over the parts only
    MxGemmArgs pp = p;
    pp.first = p.t_main;
    const dim3 g_all((unsigned)(p.t_main + (c_bf16 ? 0 : tail * p.split))), g_parts((unsigned)(tail * p.split));
#define NVFP4_MXG(E, BF)                                                                                  \
    do {                                                                                                  \
        if (exact && full) {                                                                              \
            if (g_all.x) hipLaunchKernelGGL((k_mx_gemm_exact_full<E, BF>), g_all, dim3(256), 0, s, p);    \
            if (BF && tail) hipLaunchKernelGGL((k_mx_gemm_exact_full<E, false>), g_parts, dim3(256), 0, s, pp); \
        } else if (exact) {                                                                               \
            hipLaunchKernelGGL((k_mx_gemm_exact<E, BF>), grid, dim3(256), 0, s, p);                       \
        } else if (full) {                                                                                \
            if (g_all.x) hipLaunchKernelGGL((k_mx_gemm_full8<E, BF>), g_all, dim3(512), 0, s, p);         \
            if (BF && tail) hipLaunchKernelGGL((k_mx_gemm_full8<E, false>), g_parts, dim3(512), 0, s, pp); \
        } else {                                                                                          \
            hipLaunchKernelGGL((k_mx_gemm<E, BF>), grid, dim3(256), 0, s, p);                             \
        }                                                                                                 \
    } while (0)
    if (elem == kMxE4M3) {
        if (c_bf16) NVFP4_MXG(kMxE4M3, true); else NVFP4_MXG(kMxE4M3, false);
    } else {
        if (c_bf16) NVFP4_MXG(kMxE2M1, true); else NVFP4_MXG(kMxE2M1, false);
    }
#undef NVFP4_MXG
    if (tail > 0) {
        const dim3 g2((unsigned)tail, kMxTile / 16);
        if (c_bf16) hipLaunchKernelGGL(k_mx_tail_sum<true>, g2, dim3(256), 0, s, p);
        else hipLaunchKernelGGL(k_mx_tail_sum<false>, g2, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace nvfp4
