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
// 256 FP32 accumulators per lane).  Every thread stages one A row and one B
// row: it loads the rows' 32 code bytes and 4 scale bytes per 64-wide K step
// into registers, at least two steps before use, and dequantizes the step
// after the current one into the other LDS stage (FP4 unpack instruction,
// round-toward-zero pack -- exact here -- and one packed FP16 multiply by the
// block multiplier).  The current step runs as four 16-wide K substeps of 16
// MFMAs per wave, and the dequantization is cut into 16 two-element pieces
// per substep that issue between those MFMAs (one wave per SIMD: the same
// wave has to keep the matrix core and the VALU busy, and without the
// interleave the two ran one after the other); sched_barrier pins that order.
// One workgroup barrier per step.  Loads and dequantization are branch-free
// in the loop: steps past the end are clamped re-reads, and the blocks of a
// partial last step read an in-range block with its multiplier forced to 0.
// Each operand element is expanded once per workgroup.  LDS: 2 stages x (A, B)
// x 256 rows x 144 bytes (64 FP16 + 16 bytes of padding that spreads the row
// starts over the banks).
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
    uint32_t sc;   // scale bytes of the four 16-element blocks (byte q = block q)
};

// The staged row of one operand: its code row and its scale row.
struct RowSrc {
    const uint8_t* codes;   // row start (K/2 bytes)
    const uint8_t* scales;  // first scale byte of the row (1D) or of its 16-row band (2D)
};

__device__ __forceinline__ RowSrc row_src(const Operand& op, int64_t row, int64_t K) {
    RowSrc r;
    r.codes = op.codes + row * (K / 2);
    r.scales = op.scales + (op.scale_2d ? (row / 16) : row) * (K / 16);
    return r;
}

// K step kc (0 <= kc < number of steps) of a staged row.  FAST: K % 64 == 0
// and the scale rows are 4-byte aligned, so a step is two 16-byte code loads
// and one 4-byte scale load.  Otherwise each 16-element block is loaded on its
// own; blocks past K re-read the last valid block with multiplier byte 0, so
// they dequantize to zeros.
template <bool FAST>
__device__ __forceinline__ RowStep load_row_step(const RowSrc& src, int64_t K, int64_t kc) {
    RowStep r;
    if (FAST) {
        const uint8_t* cp = src.codes + kc * (kBK / 2);
        r.c0 = *reinterpret_cast<const uint4*>(cp);
        r.c1 = *reinterpret_cast<const uint4*>(cp + 16);
        r.sc = *reinterpret_cast<const uint32_t*>(src.scales + kc * (kBK / 16));
    } else {
        const int64_t nkb = K / 16, kb0 = kc * (kBK / 16);
        uint32_t w[8];
        r.sc = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t kb = kb0 + q;
            const int64_t kbl = kb < nkb ? kb : nkb - 1;
            const uint2 t = *reinterpret_cast<const uint2*>(src.codes + 8 * kbl);
            w[2 * q] = t.x;
            w[2 * q + 1] = t.y;
            const uint32_t sb = src.scales[kbl];
            r.sc |= (kb < nkb ? sb : 0u) << (8 * q);
        }
        r.c0 = make_uint4(w[0], w[1], w[2], w[3]);
        r.c1 = make_uint4(w[4], w[5], w[6], w[7]);
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

// Dequantize 16-element block q of a RowStep into LDS row `dst` (64 FP16,
// natural K order).
__device__ __forceinline__ void store_block(const RowStep& r, int q, _Float16* dst) {
    const uint32_t wa = q == 0 ? r.c0.x : q == 1 ? r.c0.z : q == 2 ? r.c1.x : r.c1.z;
    const uint32_t wb = q == 0 ? r.c0.y : q == 1 ? r.c0.w : q == 2 ? r.c1.y : r.c1.w;
    const half2_t sc = scale_pair((r.sc >> (8 * q)) & 0xFFu);
    *reinterpret_cast<uint4*>(dst + 16 * q) = dequant8_f16(wa, sc);
    *reinterpret_cast<uint4*>(dst + 16 * q + 8) = dequant8_f16(wb, sc);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Rows of A (and the group) of the workgroup's output tile.  Grouped: tiles
// are numbered group by group, each group's rows split into 256-row tiles
// (its last one partial); tiles past the last group have ok = false.
struct TileRows {
    int64_t m0, m_end;
    int g;
    bool ok;
};

template <bool GROUPED>
__device__ __forceinline__ TileRows tile_rows(const GemmArgs& p, int64_t ty) {
    TileRows t{0, p.M, 0, true};
    if (GROUPED) {
        int64_t r = ty;
        t.ok = false;
        for (int gg = 0; gg < p.G; ++gg) {
            const int64_t lo = min(max(p.offsets[gg], (int64_t)0), p.M);
            const int64_t hi = min(max(p.offsets[gg + 1], lo), p.M);
            const int64_t tiles = (hi - lo + kBM - 1) / kBM;
            if (r < tiles) {
                t.g = gg;
                t.m_end = hi;
                t.m0 = lo + r * kBM;
                t.ok = true;
                break;
            }
            r -= tiles;
        }
    } else {
        t.m0 = ty * kBM;
    }
    return t;
}

// Row of B staged as tile row r (0..255), clamped into range.  SwiGLU: tile
// rows 0..127 are gate rows j0 + r and 128..255 the matching up rows F + j0 + r
// of the group's 2F weight rows.
template <bool SWIGLU>
__device__ __forceinline__ int64_t b_row(const GemmArgs& p, int64_t bbase, int r, int64_t tx) {
    const int64_t Ng = p.N;
    if (SWIGLU) {
        const int64_t F = Ng / 2, j0 = tx * (kBN / 2);
        const int64_t c = min(j0 + (r & 127), F - 1);
        return bbase + (r < 128 ? c : F + c);
    }
    return bbase + min(tx * kBN + r, Ng - 1);
}

// LDS tile row of B that MFMA column tile j of wave column wn reads.
template <bool SWIGLU>
__device__ __forceinline__ int b_tile_row(int wn, int j) {
    return SWIGLU ? ((j < 2 ? 0 : 128) + 64 * wn + 32 * (j & 1)) : 128 * wn + 32 * j;
}

// The lane index computed afresh (from an opaque all-ones mask), so that
// nothing lane-derived is held through a K loop for the epilogue.
__device__ __forceinline__ int fresh_lane_id() {
    uint32_t ones = ~0u;
    asm volatile("" : "+s"(ones));
    return (int)__builtin_amdgcn_mbcnt_hi(ones, __builtin_amdgcn_mbcnt_lo(ones, 0u));
}

// h = g sigma(g) u in binary32, with the hardware's base-2 exponential and
// reciprocal (each within about a unit in the last place): sigma(g) =
// 1 / (1 + 2^(-g log2 e)), 0 once the power overflows (g below about -88.7).
__device__ __forceinline__ float swiglu_h(float gt, float up) {
    const float e = __builtin_amdgcn_exp2f(gt * -1.44269504088896341f);
    return gt * __builtin_amdgcn_rcpf(1.0f + e) * up;
}

// Scale by the two tensor scales and write the wave's 128 x 128 tile (or, for
// SwiGLU, its 128 x 64 gate/up pairs) of C.  Accumulator r of MFMA tile
// (i, j) holds row 32i + 8(r/4) + 4h + r%4, column 32j + l32 of the wave tile.
//
// A wave tile wholly inside C goes out through store_wave_block; edge tiles
// take per-element bounds checks.  SwiGLU's amax: rounding to BF16 is
// monotonic, so the largest |h| rounded once is the largest rounded |h|.
template <bool GROUPED, bool SWIGLU, bool OUT_BF16>
__device__ __forceinline__ void epilogue(const GemmArgs& p, float16_t (&acc)[4][4], float alpha, int64_t m0,
                                         int64_t m_end, int wm, int wn, int lane, int64_t tx) {
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t Ng = p.N;
    const int64_t mw = m0 + 128 * wm;
    if (SWIGLU) {
        uint16_t* C = static_cast<uint16_t*>(p.C);
        const int64_t F = Ng / 2, jw = tx * (kBN / 2) + 64 * wn;
        float amax = 0.0f;
        if (mw + 128 <= m_end && jw + 64 <= F &&
            store_wave_block<4, 2, true>(C, p.ldc, mw, jw, h, l32, [&](int i, int jj, int r) {
                const float hv = swiglu_h(alpha * acc[i][jj][r], alpha * acc[i][jj + 2][r]);
                amax = fmaxf(amax, fabsf(hv));
                return hv;
            })) {
            amax = __uint_as_float(f32_to_bf16_rne(amax) << 16);
        } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int64_t c = jw + 32 * jj + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t m = mw + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (m < m_end && c < F) {
                        const float hv = swiglu_h(alpha * acc[i][jj][r], alpha * acc[i][jj + 2][r]);
                        const uint32_t b = f32_to_bf16_rne(hv);
                        C[m * p.ldc + c] = (uint16_t)b;
                        amax = fmaxf(amax, fabsf(__uint_as_float(b << 16)));
                    }
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
    const int64_t nw = tx * kBN + 128 * wn;
    if (mw + 128 <= m_end && nw + 128 <= Ng &&
        store_wave_block<4, 4, OUT_BF16>(p.C, p.ldc, mw, nw, h, l32,
                                         [&](int i, int j, int r) { return alpha * acc[i][j][r]; }))
        return;
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

template <bool GROUPED, bool SWIGLU, bool OUT_BF16, bool FAST>
__global__ void __launch_bounds__(256, 1) k_gemm(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) _Float16 smem[2][2][kBM][kLdsK];
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const TileRows tr = tile_rows<GROUPED>(p, blockIdx.y);
    if (!tr.ok) return;  // uniform across the workgroup
    const int64_t m0 = tr.m0, m_end = tr.m_end;
    const int g = tr.g;
    const int64_t K = p.K;
    const int64_t bbase = GROUPED ? (int64_t)g * p.N : 0;

    // ---- the A row and B row this thread stages ----
    const int64_t arow = min(m0 + tid, m_end - 1);
    const int64_t brow = b_row<SWIGLU>(p, bbase, tid, blockIdx.x);

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nsteps = (K + kBK - 1) / kBK;
    const RowSrc sa = row_src(p.A, arow, K), sb = row_src(p.B, brow, K);

    // LDS rows read by this wave's MFMA tiles (A: 4 tiles of 32 rows; B likewise)
    int brow_lds[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) brow_lds[j] = b_tile_row<SWIGLU>(wn, j);

    if (nsteps > 0) {  // K == 0: the accumulators stay zero
        // The loop runs K steps four at a time.  Staged rows live in two
        // register sets of two steps each: while one set's steps are being
        // dequantized (one step ahead of the MFMAs), the other set's loads are
        // in flight, issued at least two steps before their first use.  The
        // sets swap roles every two steps, so the unrolled body has static
        // register names and no copies.  A step count that is not a multiple
        // of 4 gets leading all-zero steps (scale bytes forced to 0: they
        // dequantize to zeros and add nothing).  Step j covers K step j - pad.
        const int64_t pad = (4 - nsteps % 4) % 4, nj = nsteps + pad, last = nsteps - 1;
        auto load_j = [&](const RowSrc& src, int64_t j) {
            const int64_t kc = j - pad;
            RowStep r = load_row_step<FAST>(src, K, kc < 0 ? 0 : (kc > last ? last : kc));
            if (kc < 0) r.sc = 0u;
            return r;
        };
        struct TwoSteps {
            RowStep a0, b0, a1, b1;  // A row and B row of the first and second step
        };
        auto load2 = [&](TwoSteps& t, int64_t j) {
            t.a0 = load_j(sa, j);
            t.b0 = load_j(sb, j);
            t.a1 = load_j(sa, j + 1);
            t.b1 = load_j(sb, j + 1);
        };
        {
            const RowStep ra = load_j(sa, 0), rb = load_j(sb, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                store_block(ra, q, &smem[0][0][tid][0]);
                store_block(rb, q, &smem[0][1][tid][0]);
            }
        }
        TwoSteps P, Q;
        load2(P, 1);
        load2(Q, 3);
        __syncthreads();

        // One step: MFMAs from LDS stage j & 1 while da/db (step j + 1) are
        // dequantized into the other stage.  Per 16-wide substep the
        // wave's 16 MFMAs alternate with the 16 two-element dequantization
        // pieces of block s of both staged rows (3 VALU each), the next
        // substep's 8 fragment reads go out after the third MFMA, and each
        // completed 8-element group is written to LDS; sched_barrier(0) keeps
        // that order.
        auto step = [&](int64_t j, const RowStep& da, const RowStep& db) {
            const int st = (int)(j & 1);
            half8_t fr[2][8];  // [set][A0..A3, B0..B3]
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fr[0][i] = *reinterpret_cast<const half8_t*>(&smem[st][0][128 * wm + 32 * i + l32][8 * h]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fr[0][4 + j] = *reinterpret_cast<const half8_t*>(&smem[st][1][brow_lds[j] + l32][8 * h]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int cur = s & 1, nxt = cur ^ 1;
                const uint32_t wsrc[4] = {
                    s == 0 ? da.c0.x : s == 1 ? da.c0.z : s == 2 ? da.c1.x : da.c1.z,
                    s == 0 ? da.c0.y : s == 1 ? da.c0.w : s == 2 ? da.c1.y : da.c1.w,
                    s == 0 ? db.c0.x : s == 1 ? db.c0.z : s == 2 ? db.c1.x : db.c1.z,
                    s == 0 ? db.c0.y : s == 1 ? db.c0.w : s == 2 ? db.c1.y : db.c1.w};
                const half2_t sca = scale_pair((da.sc >> (8 * s)) & 0xFFu);
                const half2_t scb = scale_pair((db.sc >> (8 * s)) & 0xFFu);
                uint32_t outw[4][4];
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int i = m >> 2, j = m & 3;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[cur][i], fr[cur][4 + j], acc[i][j], 0, 0, 0);
                    if (m == 2 && s < 3) {
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii)
                            fr[nxt][ii] = *reinterpret_cast<const half8_t*>(
                                &smem[st][0][128 * wm + 32 * ii + l32][16 * (s + 1) + 8 * h]);
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            fr[nxt][4 + jj] = *reinterpret_cast<const half8_t*>(
                                &smem[st][1][brow_lds[jj] + l32][16 * (s + 1) + 8 * h]);
                    }
                    // dequantization piece m: word m / 4, code pair m % 4
                    const int wq = m >> 2, pq = m & 3;
                    const float2 f = e2m1x2_unpack(wsrc[wq], pq);
                    const half2_t hv = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(f.x, f.y));
                    outw[wq][pq] = __builtin_bit_cast(uint32_t, hv * (wq < 2 ? sca : scb));
                    if (pq == 3)
                        *reinterpret_cast<uint4*>(&smem[st ^ 1][wq >> 1][tid][16 * s + 8 * (wq & 1)]) =
                            make_uint4(outw[wq][0], outw[wq][1], outw[wq][2], outw[wq][3]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            __syncthreads();
        };

        // (loads past the last step are clamped re-reads, unused)
        for (int64_t j = 0; j < nj; j += 4) {
            step(j, P.a0, P.b0);
            step(j + 1, P.a1, P.b1);
            load2(P, j + 5);
            step(j + 2, Q.a0, Q.b0);
            step(j + 3, Q.a1, Q.b1);
            load2(Q, j + 7);
        }
    }

    epilogue<GROUPED, SWIGLU, OUT_BF16>(p, acc, p.A.ts[0] * p.B.ts[GROUPED ? g : 0], m0, m_end, wm, wn, lane, blockIdx.x);
}

// ============================================================ ring kernel
// The kernel for whole 64-wide K steps and 4-byte-aligned scale rows (every
// shape of the benchmarked workloads).  Raw operands go straight from global
// memory into LDS: a ring of kRing slots, each holding one K step of both
// operands' codes (256 rows x 32 bytes) and scale bytes (256 rows x 4 bytes),
// loaded by global_load_lds (no register staging; lane i of a load lands at
// the slot base + i x size), kRing - 1 steps ahead of use.  Each wave then
// converts its own MFMA fragments straight into registers: FP4 pair -> FP16
// pair with the gfx950 convert (exact), times the block multiplier (FP8 pair
// -> FP16 pair convert, exact; the product has at most 6 significant bits).
// LDS carries 4.5 bits per element instead of 16, and no FP16 tile is written.
//
// K order inside a step: lane (l32, h) of substep s supplies elements
// K = 32 h + 8 s .. + 7 of the step (the same map on A and B, so every product
// pairs equal K; over the four substeps and both lane halves it covers the 64
// elements once).  A lane's codes for the whole step are then one 16-byte LDS
// read per fragment row, and the 64 lanes of a read cover 1 KiB contiguously.
//
// Per step, per wave: 4 substeps of 16 MFMAs; between the MFMAs of substep s
// the fragments of substep s + 1 are converted (32 two-element pieces, 2 VALU
// each).  In substep 2 the wave waits for its own loads of the next step,
// joins the workgroup barrier, reads the next step's raw fragments and issues
// the loads of the step kRing steps ahead into the slot just consumed.
constexpr int kRing = 4;
constexpr int kSlotCodes = kBM * (kBK / 2);   // 8192 bytes per operand
constexpr int kSlotScales = kBM * (kBK / 16); // 1024 bytes per operand

struct RingSlot {
    uint8_t a_codes[kSlotCodes];
    uint8_t b_codes[kSlotCodes];
    uint8_t a_sc[kSlotScales];
    uint8_t b_sc[kSlotScales];
};

typedef __attribute__((address_space(1))) void gmem_t;
typedef __attribute__((address_space(3))) void lmem_t;

// Per-thread global sources of the ring loads: code rows for tile rows
// 64 w + L/2 and 64 w + 32 + L/2 (16-byte chunk L % 2), scale rows for tile
// row 64 w + L (L = lane, w = wave).
struct RingSrc {
    const uint8_t *a0, *a1, *b0, *b1, *as, *bs;
};

__device__ __forceinline__ void ring_load(const RingSrc& rs, int64_t kc, RingSlot& slot, int w) {
    const int64_t co = kc * (kBK / 2), so = kc * (kBK / 16);
    __builtin_amdgcn_global_load_lds((gmem_t*)(rs.a0 + co), (lmem_t*)&slot.a_codes[64 * w * 32], 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(rs.a1 + co), (lmem_t*)&slot.a_codes[(64 * w + 32) * 32], 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(rs.b0 + co), (lmem_t*)&slot.b_codes[64 * w * 32], 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(rs.b1 + co), (lmem_t*)&slot.b_codes[(64 * w + 32) * 32], 16, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(rs.as + so), (lmem_t*)&slot.a_sc[64 * w * 4], 4, 0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(rs.bs + so), (lmem_t*)&slot.b_sc[64 * w * 4], 4, 0, 0);
}
constexpr int kRingLoadsPerStep = 6;

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations of this wave are outstanding, leaving the other counters.
constexpr unsigned vmcnt_at_most(unsigned n) {
    return (n & 15u) | ((n >> 4) << 14) | (7u << 4) | (15u << 8);
}

// A wave's raw fragments of one step: codes of its 4 A and 4 B fragment rows
// (32 codes each), their two scale bytes, and (after scale_frags) the two
// block multipliers as an FP16 pair.
struct RawFrags {
    uint4 c[8];       // A0..A3, B0..B3
    uint32_t sb[8];   // scale bytes of blocks 2h, 2h + 1
    half2_t sc[8];
    bool zero;        // a leading padding step: multipliers forced to 0
};

__device__ __forceinline__ void read_frags(const RingSlot& slot, int arow0, const int (&brow)[4], int l32,
                                           int h, bool zero, RawFrags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = arow0 + 32 * i + l32;
        f.c[i] = *reinterpret_cast<const uint4*>(&slot.a_codes[r * 32 + 16 * h]);
        f.sb[i] = *reinterpret_cast<const uint16_t*>(&slot.a_sc[r * 4 + 2 * h]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = brow[j] + l32;
        f.c[4 + j] = *reinterpret_cast<const uint4*>(&slot.b_codes[r * 32 + 16 * h]);
        f.sb[4 + j] = *reinterpret_cast<const uint16_t*>(&slot.b_sc[r * 4 + 2 * h]);
    }
    f.zero = zero;
}

// Block multipliers of the fragments: FP8 pair -> FP16 pair (exact).
__device__ __forceinline__ void scale_frags(RawFrags& f) {
#pragma unroll
    for (int o = 0; o < 8; ++o)
        f.sc[o] = __builtin_bit_cast(half2_t,
                                     __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.zero ? 0u : f.sb[o], 1.0f, false));
}

// Piece p (0..3) of fragment o for substep s: codes 2p, 2p+1 of the substep's
// 8 -> one FP16 pair times the block multiplier.
__device__ __forceinline__ uint32_t frag_piece(const RawFrags& f, int o, int s, int p) {
    const uint4& c = f.c[o];
    const uint32_t w = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
    half2_t v;
    switch (p) {
        case 0: v = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)); break;
        case 1: v = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)); break;
        case 2: v = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)); break;
        default: v = __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)); break;
    }
    const _Float16 m = s < 2 ? f.sc[o].x : f.sc[o].y;  // block 2h (s = 0, 1) or 2h + 1
    return __builtin_bit_cast(uint32_t, v * m);
}

template <bool GROUPED, bool SWIGLU, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1) k_gemm_ring(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) RingSlot ring0, ring1, ring2, ring3;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const TileRows tr = tile_rows<GROUPED>(p, blockIdx.y);
    if (!tr.ok) return;  // uniform across the workgroup
    const int64_t m0 = tr.m0, m_end = tr.m_end;
    const int g = tr.g;
    const int64_t K = p.K;
    const int64_t bbase = GROUPED ? (int64_t)g * p.N : 0;

    RingSrc rs;
    {
        const int r0 = 64 * w + (lane >> 1), r1 = r0 + 32, rsc = 64 * w + lane;
        const int64_t chunk = 16 * (lane & 1);
        const RowSrc a0 = row_src(p.A, min(m0 + r0, m_end - 1), K);
        const RowSrc a1 = row_src(p.A, min(m0 + r1, m_end - 1), K);
        const RowSrc b0 = row_src(p.B, b_row<SWIGLU>(p, bbase, r0, blockIdx.x), K);
        const RowSrc b1 = row_src(p.B, b_row<SWIGLU>(p, bbase, r1, blockIdx.x), K);
        rs.a0 = a0.codes + chunk;
        rs.a1 = a1.codes + chunk;
        rs.b0 = b0.codes + chunk;
        rs.b1 = b1.codes + chunk;
        rs.as = row_src(p.A, min(m0 + rsc, m_end - 1), K).scales;
        rs.bs = row_src(p.B, b_row<SWIGLU>(p, bbase, rsc, blockIdx.x), K).scales;
    }
    const int arow0 = 128 * wm;
    int brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) brow[j] = b_tile_row<SWIGLU>(wn, j);

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t nsteps = K / kBK;
    if (nsteps > 0) {  // K == 0: the accumulators stay zero
        // Steps run four at a time (ring slots and fragment buffers then have
        // static names); a step count that is not a multiple of 4 gets leading
        // steps whose multipliers are forced to 0.  Step j covers K step j - pad.
        const int64_t pad = (4 - nsteps % 4) % 4, nj = nsteps + pad, last = nsteps - 1;
        auto kc_of = [&](int64_t j) {
            const int64_t kc = j - pad;
            return kc < 0 ? (int64_t)0 : (kc > last ? last : kc);
        };
        ring_load(rs, kc_of(0), ring0, w);
        ring_load(rs, kc_of(1), ring1, w);
        ring_load(rs, kc_of(2), ring2, w);
        ring_load(rs, kc_of(3), ring3, w);
        // step 0 landed (three later steps may be outstanding), then the barrier
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(3 * kRingLoadsPerStep));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");

        RawFrags fx, fy;            // raw fragments of the current / next step (alternating)
        uint32_t op[2][8][4];       // converted fragments, double-buffered by substep
        read_frags(ring0, arow0, brow, l32, h, pad > 0, fx);
        scale_frags(fx);
#pragma unroll
        for (int o = 0; o < 8; ++o)
#pragma unroll
            for (int q = 0; q < 4; ++q) op[0][o][q] = frag_piece(fx, o, 0, q);

        auto step = [&](int64_t j, RingSlot& cur, RingSlot& nxt, RawFrags& fc, RawFrags& fn) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int ob = s & 1;
                if (s == 2) {
                    // own loads of step j + 1 done (steps j + 2, j + 3 may be
                    // in flight), workgroup barrier: every wave's part of step
                    // j + 1 is in LDS and every wave is done reading `cur`
                    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(2 * kRingLoadsPerStep));
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    read_frags(nxt, arow0, brow, l32, h, j + 1 < pad, fn);
                    ring_load(rs, kc_of(j + 4), cur, w);
                }
                if (s == 3) scale_frags(fn);  // first use of the next step's fragments
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const int i = m >> 2, jj = m & 3;
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(half8_t, op[ob][i]), __builtin_bit_cast(half8_t, op[ob][4 + jj]),
                        acc[i][jj], 0, 0, 0);
                    // two conversion pieces for the next substep (or step)
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int piece = 2 * m + u, o = piece >> 2, q = piece & 3;
                        op[ob ^ 1][o][q] = s < 3 ? frag_piece(fc, o, s + 1, q) : frag_piece(fn, o, 0, q);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        for (int64_t j = 0; j < nj; j += 4) {
            step(j, ring0, ring1, fx, fy);
            step(j + 1, ring1, ring2, fy, fx);
            step(j + 2, ring2, ring3, fx, fy);
            step(j + 3, ring3, ring0, fy, fx);
        }
        // the last steps' look-ahead loads (clamped re-reads into slots nobody
        // reads again) must land before the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    }
    epilogue<GROUPED, SWIGLU, OUT_BF16>(p, acc, p.A.ts[0] * p.B.ts[GROUPED ? g : 0], m0, m_end, wm, wn, fresh_lane_id(), blockIdx.x);
}

// ============================================================ full-line kernel
// For K % 512 == 0 with 16-byte-aligned scale rows (every benchmarked shape):
// the ring kernel's tile, fragment conversion and MFMA interleave, with the
// operands moved in whole cache lines.  Each distinct line a wave-wide load
// touches costs about the same whatever part of it is used, and the ring
// kernel's 32-byte code and 4-byte scale pieces per row and step made the
// loads 12% of its time.  Here a slot holds 128 bytes of codes per tile row
// (256 K elements, 4 K steps) and that chunk's 16 scale bytes per row -- one
// 16-byte load per row -- for both operands; two slots, the next chunk's loads
// in flight during a whole chunk (4 steps of 64 MFMAs), one barrier per chunk.
// 16-byte code chunk c of slot row r sits at chunk c ^ (r % 8) ^ ((r / 8) % 4)
// (row bits 0..4; fragment rows 32 apart share it), which spreads the
// fragment reads over every bank.
constexpr int kFullCodes = kBM * 128;  // code bytes per operand per slot
constexpr int kFullSc = kBM * 16;      // scale bytes per operand per slot

// One ring slot: four separate LDS arrays (A codes, B codes, A scales, B
// scales).  Declared per slot as distinct variables, so the compiler can tell
// the slot being read from the one in-flight loads target; the same-operand
// arrays of the two slots end up 32 KiB (codes) or 4 KiB (scales) apart, so
// one address register per fragment row serves both slots through the LDS
// instruction's immediate offset.
struct FullSlot {
    uint8_t* a_codes;
    uint8_t* b_codes;
    uint8_t* a_sc;
    uint8_t* b_sc;
};

__device__ __forceinline__ int full_swz(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// Wave-uniform bases and 32-bit per-lane byte offsets of the chunk-0 sources:
// code loads t = 0..7 (tile rows 64 w + 8 t + L / 8, chunk L % 8), scale rows
// 64 w + L.
struct FullSrc {
    const uint8_t *ac, *bc, *as, *bs;
    uint32_t a[8], b[8];
    uint32_t sa, sb;
};
constexpr int kFullLoadsPerChunk = 18;

__device__ __forceinline__ void full_load(const FullSrc& src, int64_t chunk, const FullSlot& slot, int w) {
    const uint8_t* ac = src.ac + chunk * 128;
    const uint8_t* bc = src.bc + chunk * 128;
#pragma unroll
    for (int t = 0; t < 8; ++t)
        __builtin_amdgcn_global_load_lds((gmem_t*)(ac + src.a[t]), (lmem_t*)(slot.a_codes + (64 * w + 8 * t) * 128), 16,
                                         0, 0);
#pragma unroll
    for (int t = 0; t < 8; ++t)
        __builtin_amdgcn_global_load_lds((gmem_t*)(bc + src.b[t]), (lmem_t*)(slot.b_codes + (64 * w + 8 * t) * 128), 16,
                                         0, 0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.as + chunk * 16 + src.sa), (lmem_t*)(slot.a_sc + 64 * w * 16), 16, 0,
                                     0);
    __builtin_amdgcn_global_load_lds((gmem_t*)(src.bs + chunk * 16 + src.sb), (lmem_t*)(slot.b_sc + 64 * w * 16), 16, 0,
                                     0);
}

// Raw fragments of K step t (0..3) of a chunk: lane (l32, h) takes the
// step's codes K = 32 h .. 32 h + 31 (logical chunk 2 t + h) and the scale
// bytes of blocks 2 h, 2 h + 1, as in the ring kernel.
__device__ __forceinline__ void full_read_frags(const FullSlot& slot, int t, int arow0, const int (&brow)[4], int l32,
                                                int h, RawFrags& f) {
    const int pc = (2 * t + h) ^ full_swz(l32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = arow0 + 32 * i + l32;
        f.c[i] = *reinterpret_cast<const uint4*>(&slot.a_codes[r * 128 + 16 * pc]);
        f.sb[i] = *reinterpret_cast<const uint16_t*>(&slot.a_sc[r * 16 + 4 * t + 2 * h]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = brow[j] + l32;
        f.c[4 + j] = *reinterpret_cast<const uint4*>(&slot.b_codes[r * 128 + 16 * pc]);
        f.sb[4 + j] = *reinterpret_cast<const uint16_t*>(&slot.b_sc[r * 16 + 4 * t + 2 * h]);
    }
    f.zero = false;
}

// Fragment o (0..3: A tiles, 4..7: B tiles) of full_read_frags, on its own.
__device__ __forceinline__ void full_read_frag(const FullSlot& slot, int t, int arow0, const int (&brow)[4], int l32,
                                               int h, int o, RawFrags& f) {
    const int pc = (2 * t + h) ^ full_swz(l32);
    if (o < 4) {
        const int r = arow0 + 32 * o + l32;
        f.c[o] = *reinterpret_cast<const uint4*>(&slot.a_codes[r * 128 + 16 * pc]);
        f.sb[o] = *reinterpret_cast<const uint16_t*>(&slot.a_sc[r * 16 + 4 * t + 2 * h]);
    } else {
        const int r = brow[o - 4] + l32;
        f.c[o] = *reinterpret_cast<const uint4*>(&slot.b_codes[r * 128 + 16 * pc]);
        f.sb[o] = *reinterpret_cast<const uint16_t*>(&slot.b_sc[r * 16 + 4 * t + 2 * h]);
    }
    f.zero = false;
}

// Work item L = first + blockIdx.x (tiles numbered row-major over a
// tiles_x-wide grid of 256 x 256 tiles): tiles 0 .. t_main - 1 whole, one
// per workgroup; the tiles after them (a last round that would leave most
// compute units idle) each split `split` ways along K, part s taking chunk
// pairs [s P / split, (s + 1) P / split) of the P = K / 512 pairs.  A part
// writes its raw binary32 accumulators to `partials` (part j of the tail at
// float4 index (64 j + e) 256 + thread, e = 0..63: coalesced across the
// workgroup); k_gemm_tail_sum adds them up and writes the tile.
struct FullWork {
    int tile;
    int part;  // -1: the whole tile
    int64_t c0, c1;
};

__device__ __forceinline__ FullWork full_work(int first, int t_main, int split, int64_t nchunks) {
    FullWork wk{first + (int)blockIdx.x, -1, 0, nchunks};
    if (wk.tile >= t_main) {
        const int j = wk.tile - t_main, s = j % split;
        const int64_t pairs = nchunks / 2;
        wk.tile = t_main + j / split;
        wk.part = j;
        wk.c0 = 2 * (s * pairs / split);
        wk.c1 = 2 * ((s + 1) * pairs / split);
    }
    return wk;
}

template <bool GROUPED, bool SWIGLU, bool OUT_BF16>
__global__ void __launch_bounds__(256, 1) k_gemm_full(GemmArgs p, int tiles_x, int first, int t_main, int split,
                                                      float* __restrict__ partials) {
    __shared__ __attribute__((aligned(16))) uint8_t a0c[kFullCodes];
    __shared__ __attribute__((aligned(16))) uint8_t a1c[kFullCodes];
    __shared__ __attribute__((aligned(16))) uint8_t b0c[kFullCodes];
    __shared__ __attribute__((aligned(16))) uint8_t b1c[kFullCodes];
    __shared__ __attribute__((aligned(16))) uint8_t a0s[kFullSc];
    __shared__ __attribute__((aligned(16))) uint8_t a1s[kFullSc];
    __shared__ __attribute__((aligned(16))) uint8_t b0s[kFullSc];
    __shared__ __attribute__((aligned(16))) uint8_t b1s[kFullSc];
    const FullSlot slot0{a0c, b0c, a0s, b0s}, slot1{a1c, b1c, a1s, b1s};
    const int tid = threadIdx.x;
    // the wave index is uniform: held in a scalar register, the LDS
    // destinations of the loads need no vector registers
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // (the two forms of the lane index are equal; with either one alone, one
    // of the SwiGLU instances got a dead register spill from the allocator)
    const int lane = GROUPED ? (int)__lane_id() : (tid & 63);
    const int wm = w >> 1, wn = w & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int64_t K = p.K, kc2 = K / 2, ks = K / 16;
    const int64_t nchunks = K / 256;  // even: K % 512 == 0
    const FullWork wk = full_work(first, t_main, split, nchunks);  // uniform across the workgroup
    const int64_t tx = wk.tile % tiles_x, ty = wk.tile / tiles_x;
    const TileRows tr = tile_rows<GROUPED>(p, ty);
    if (!tr.ok) return;  // uniform across the workgroup
    const int64_t m0 = tr.m0, m_end = tr.m_end;
    const int g = tr.g;
    const int64_t bbase = GROUPED ? (int64_t)g * p.N : 0;

    FullSrc src;
    src.ac = p.A.codes + m0 * kc2;
    src.bc = p.B.codes + bbase * kc2;
    src.as = p.A.scales;
    src.bs = p.B.scales;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int r = 64 * w + 8 * t + (lane >> 3);
        const int c = (lane & 7) ^ full_swz(r);  // the swizzle is an involution
        src.a[t] = (uint32_t)((min(m0 + r, m_end - 1) - m0) * kc2 + 16 * c);
        src.b[t] = (uint32_t)((b_row<SWIGLU>(p, bbase, r, tx) - bbase) * kc2 + 16 * c);
    }
    {
        const int r = 64 * w + lane;
        const int64_t ga = min(m0 + r, m_end - 1), gb = b_row<SWIGLU>(p, bbase, r, tx);
        src.sa = (uint32_t)((p.A.scale_2d ? ga / 16 : ga) * ks);
        src.sb = (uint32_t)((p.B.scale_2d ? gb / 16 : gb) * ks);
    }
    const int arow0 = 128 * wm;
    int brow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) brow[j] = b_tile_row<SWIGLU>(wn, j);

    float16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int64_t c0 = wk.c0, c1 = wk.c1;
    auto cclamp = [&](int64_t c) { return c < c1 ? c : c1 - 1; };
    full_load(src, c0, slot0, w);
    full_load(src, c0 + 1, slot1, w);
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kFullLoadsPerChunk));  // chunk 0 landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    RawFrags fx, fy;            // raw fragments of the current / next step (alternating)
    uint32_t op[2][8][4];       // converted fragments, double-buffered by substep
    full_read_frags(slot0, 0, arow0, brow, l32, h, fx);
    scale_frags(fx);
#pragma unroll
    for (int o = 0; o < 8; ++o)
#pragma unroll
        for (int q = 0; q < 4; ++q) op[0][o][q] = frag_piece(fx, o, 0, q);

    // K step t (0..3) of the chunk in `cur`; `other` holds the next chunk
    auto step = [&](int64_t chunk, int t, const FullSlot& cur, const FullSlot& other, RawFrags& fc, RawFrags& fn) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int ob = s & 1;
            if (s == 2) {
                if (t == 3) {
                    // the next chunk's loads landed; after the barrier every
                    // wave has read all of `cur`, which takes chunk + 2
                    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
                    asm volatile("" ::: "memory");
                    __builtin_amdgcn_s_barrier();
                    asm volatile("" ::: "memory");
                    full_load(src, cclamp(chunk + 2), cur, w);
                }
            }
            if (s == 3) scale_frags(fn);  // first use of the next step's fragments
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const int i = m >> 2, jj = m & 3;
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(half8_t, op[ob][i]), __builtin_bit_cast(half8_t, op[ob][4 + jj]),
                    acc[i][jj], 0, 0, 0);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int piece = 2 * m + u, o = piece >> 2, q = piece & 3;
                    op[ob ^ 1][o][q] = s < 3 ? frag_piece(fc, o, s + 1, q) : frag_piece(fn, o, 0, q);
                }
                // the next step's fragments, one per MFMA over the first half of substep 2
                if (s == 2 && m < 8) {
                    if (t == 3) full_read_frag(other, 0, arow0, brow, l32, h, m, fn);
                    else full_read_frag(cur, t + 1, arow0, brow, l32, h, m, fn);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    for (int64_t ch = c0; ch < c1; ch += 2) {
        step(ch, 0, slot0, slot1, fx, fy);
        step(ch, 1, slot0, slot1, fy, fx);
        step(ch, 2, slot0, slot1, fx, fy);
        step(ch, 3, slot0, slot1, fy, fx);
        step(ch + 1, 0, slot1, slot0, fx, fy);
        step(ch + 1, 1, slot1, slot0, fy, fx);
        step(ch + 1, 2, slot1, slot0, fx, fy);
        step(ch + 1, 3, slot1, slot0, fy, fx);
    }
    // the last look-ahead loads (clamped re-reads) land before the LDS is released
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));
    // the tile's rows and group found again rather than kept through the loop
    // (held there, they cost the grouped SwiGLU instance a spilled register)
    const TileRows te = tile_rows<GROUPED>(p, ty);
    GemmArgs q = p;
    float alpha = p.A.ts[0] * p.B.ts[GROUPED ? te.g : 0];
    int64_t em0 = te.m0, em_end = te.m_end, etx = tx;
    if constexpr (!GROUPED && !SWIGLU && !OUT_BF16) {
        if (wk.part >= 0) {
            // a part: its raw sums as a 256 x 256 binary32 matrix, through
            // the same epilogue (one code path for the allocator)
            q.C = partials + (int64_t)wk.part * kBM * kBN;
            q.ldc = kBN;
            q.N = kBN;
            alpha = 1.0f;
            em0 = 0;
            em_end = kBM;
            etx = 0;
        }
    }
    epilogue<GROUPED, SWIGLU, OUT_BF16>(q, acc, alpha, em0, em_end, wm, wn, fresh_lane_id(), etx);
}

// The tail tiles of a split k_gemm_full launch: element (r, c) of tile
// t_main + blockIdx.x is alpha times the sum of its parts' element (r, c),
// added in part order (deterministic), rounded to BF16 as the epilogue
// rounds for BF16 outputs.
// Workgroup (x, y) covers 16 rows from 16 y of the tile.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) k_gemm_tail_sum(GemmArgs p, int tiles_x, int t_main, int split,
                                                       const float* __restrict__ partials) {
    const int tile = t_main + (int)blockIdx.x;
    const int64_t m0 = (int64_t)(tile / tiles_x) * kBM, n0 = (int64_t)(tile % tiles_x) * kBN;
    const float alpha = p.A.ts[0] * p.B.ts[0];
    const float* part0 = partials + (int64_t)blockIdx.x * split * kBM * kBN;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int e = 4 * (256 * k + threadIdx.x);  // first of 4 elements in 16 rows x 256
        const int r = 16 * blockIdx.y + e / kBN, c = e % kBN;
        float4 v = *reinterpret_cast<const float4*>(part0 + r * kBN + c);
        for (int s = 1; s < split; ++s) {
            const float4 u = *reinterpret_cast<const float4*>(part0 + (int64_t)s * kBM * kBN + r * kBN + c);
            v.x += u.x;
            v.y += u.y;
            v.z += u.z;
            v.w += u.w;
        }
        const int64_t m = m0 + r;
        if (m >= p.M) continue;
        const float o[4] = {alpha * v.x, alpha * v.y, alpha * v.z, alpha * v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + c + q;
            if (n >= p.N) break;
            if (OUT_BF16)
                static_cast<uint16_t*>(p.C)[m * p.ldc + n] = (uint16_t)f32_to_bf16_rne(o[q]);
            else
                static_cast<float*>(p.C)[m * p.ldc + n] = o[q];
        }
    }
}

__global__ void k_zero_float(float* p) {
    if (threadIdx.x == 0) p[0] = 0.0f;
}

namespace {
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Whole 64-wide steps and 4-byte-aligned scale rows: the two-load step reader.
inline bool fast_path(const Operand& A, const Operand& B, int64_t K) {
    return K % kBK == 0 && (reinterpret_cast<uintptr_t>(A.scales) & 3) == 0 &&
           (reinterpret_cast<uintptr_t>(B.scales) & 3) == 0;
}

// The full-line kernel: 512-multiple K, 16-byte-aligned scale rows, per-lane
// byte offsets that fit 32 bits (B's rows of one group and either operand's
// scale rows), and a tile count that fits its one-dimensional grid.
inline bool full_path(const Operand& A, const Operand& B, int64_t a_rows, int64_t b_rows, int64_t K,
                      int64_t tiles) {
    const uint64_t lim = (uint64_t)1 << 32;
    return K > 0 && K % 512 == 0 && (reinterpret_cast<uintptr_t>(A.scales) & 15) == 0 &&
           (reinterpret_cast<uintptr_t>(B.scales) & 15) == 0 && (uint64_t)b_rows * (uint64_t)(K / 2) < lim &&
           (uint64_t)a_rows * (uint64_t)(K / 16) < lim && (uint64_t)b_rows * (uint64_t)(K / 16) < lim &&
           tiles <= INT32_MAX / 8;
}

// Bytes of one tile part's accumulators.
constexpr int64_t kPartBytes = (int64_t)kBM * kBN * 4;
}  // namespace

GemmSplit gemm_split_plan(int64_t M, int64_t N, int64_t K, bool swiglu, int cus) {
    GemmSplit sp{0, 1, 0};
    if (swiglu || M <= 0 || N <= 0 || K <= 0 || K % 512 || cus <= 0) return sp;
    const int64_t tiles = cdiv(N, kBN) * cdiv(M, kBM), tail = tiles % cus;
    sp.t_main = tiles;
    if (tail == 0) return sp;
    // the last round's tiles, each split over the compute units they leave
    // idle, every part at least one unit of 512 K (a pair of 256-element
    // chunks).  A split into q parts ends with its longest part, ceil(U / q)
    // of the U units, so it saves U - ceil(U / q) units of a lone tile's time
    // (about 8.5 µs per unit, measured on single rounds of 9 tiles at K =
    // 1024 and 2048); it costs about 1.5 µs + 2.6 µs per part plus 0.3 µs
    // per MiB of parts written and re-read (as for the MX GEMM).  The q with
    // the largest positive gain, else no split.
    const int64_t units = K / 512, smax = std::min<int64_t>(std::min<int64_t>(cus / tail, units), kMaxTailSplit);
    int64_t split = 1;
    double best = 0.0;
    for (int64_t q = 2; q <= smax; ++q) {
        const int64_t longest = (units + q - 1) / q;
        const double gain = 8.5 * (double)(units - longest) - 1.5 - 2.6 * (double)q - 0.3 * 0.25 * (double)(tail * q);
        if (gain > best) best = gain, split = q;
    }
    if (split < 2) return sp;
    sp.t_main = tiles - tail;
    sp.split = (int)split;
    sp.bytes = tail * split * kPartBytes;
    return sp;
}

hipError_t device_cus(int& cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    return e;
}

hipError_t launch_gemm(const Operand& A, const Operand& B, int64_t M, int64_t N, int64_t K,
                       void* C, bool c_bf16, int64_t ldc, bool swiglu, void* ws, size_t ws_bytes,
                       hipStream_t s) {
    if (M == 0 || N == 0) return hipSuccess;
    GemmArgs p{A, B, M, N, K, C, ldc, nullptr, 1, nullptr};
    // SwiGLU: gate column j and up column F + j share a tile, 128 output columns per tile
    const int64_t tx = swiglu ? cdiv(N / 2, kBN / 2) : cdiv(N, kBN), ty = cdiv(M, kBM);
    if (full_path(A, B, M, N, K, tx * ty)) {
        GemmSplit sp{tx * ty, 1, 0};
        if (ws && !swiglu) {
            int cus = 0;
            const hipError_t e = device_cus(cus);
            if (e != hipSuccess) return e;
            const GemmSplit plan = gemm_split_plan(M, N, K, false, cus);
            if (plan.split > 1 && (size_t)plan.bytes <= ws_bytes) sp = plan;
        }
        const int64_t tail = tx * ty - sp.t_main;
        float* parts = static_cast<float*>(ws);
        const int itx = (int)tx, tm = (int)sp.t_main, spl = sp.split;
        // the parts always run in the FP32 instance (their sums are binary32);
        // with a BF16 output the whole tiles take the BF16 instance, launched
        // first over those tiles only
        if (swiglu) {
            hipLaunchKernelGGL((k_gemm_full<false, true, true>), dim3((unsigned)(tx * ty)), dim3(256), 0, s, p, itx, 0,
                               tm, 1, nullptr);
        } else if (c_bf16) {
            if (tm > 0)
                hipLaunchKernelGGL((k_gemm_full<false, false, true>), dim3((unsigned)tm), dim3(256), 0, s, p, itx, 0,
                                   tm, 1, nullptr);
            if (tail > 0)
                hipLaunchKernelGGL((k_gemm_full<false, false, false>), dim3((unsigned)(tail * spl)), dim3(256), 0, s,
                                   p, itx, tm, tm, spl, parts);
        } else {
            hipLaunchKernelGGL((k_gemm_full<false, false, false>), dim3((unsigned)(tm + tail * spl)), dim3(256), 0, s,
                               p, itx, 0, tm, spl, parts);
        }
        if (tail > 0) {
            const dim3 g2((unsigned)tail, kBM / 16);
            if (c_bf16)
                hipLaunchKernelGGL((k_gemm_tail_sum<true>), g2, dim3(256), 0, s, p, itx, tm, spl, parts);
            else
                hipLaunchKernelGGL((k_gemm_tail_sum<false>), g2, dim3(256), 0, s, p, itx, tm, spl, parts);
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)tx, (unsigned)ty);
    if (swiglu) {
        if (fast_path(A, B, K))
            hipLaunchKernelGGL((k_gemm_ring<false, true, true>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((k_gemm<false, true, true, false>), grid, dim3(256), 0, s, p);
    } else if (fast_path(A, B, K)) {
        if (c_bf16)
            hipLaunchKernelGGL((k_gemm_ring<false, false, true>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((k_gemm_ring<false, false, false>), grid, dim3(256), 0, s, p);
    } else {
        if (c_bf16)
            hipLaunchKernelGGL((k_gemm<false, false, true, false>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((k_gemm<false, false, false, false>), grid, dim3(256), 0, s, p);
    }
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
    const int64_t tx = swiglu ? cdiv(n_per_group / 2, kBN / 2) : cdiv(n_per_group, kBN);
    const bool fast = fast_path(A, B, K);
    const bool full = full_path(A, B, total_rows, n_per_group, K, tx * mtiles);
    const dim3 grid2((unsigned)tx, (unsigned)mtiles), grid1((unsigned)(tx * mtiles));
    const int itx = (int)tx, nt = (int)(tx * mtiles);
#define NVFP4_GROUPED(SW, BF)                                                                               \
    do {                                                                                                    \
        if (full)                                                                                           \
            hipLaunchKernelGGL((k_gemm_full<true, SW, BF>), grid1, dim3(256), 0, s, p, itx, 0, nt, 1, nullptr); \
        else if (fast)                                                                                      \
            hipLaunchKernelGGL((k_gemm_ring<true, SW, BF>), grid2, dim3(256), 0, s, p);                     \
        else                                                                                                \
            hipLaunchKernelGGL((k_gemm<true, SW, BF, false>), grid2, dim3(256), 0, s, p);                   \
    } while (0)
    if (swiglu) NVFP4_GROUPED(true, true);
    else if (c_bf16) NVFP4_GROUPED(false, true);
    else NVFP4_GROUPED(false, false);
#undef NVFP4_GROUPED
    return hipGetLastError();
}

}  // namespace nvfp4
