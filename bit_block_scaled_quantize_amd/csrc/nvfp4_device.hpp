// Device-side building blocks of the NVFP4 kernels for gfx950 (CDNA4).
//
// The number format and rounding rules implemented here are the ones fixed in
// include/nvfp4.h: E2M1 elements ("Nvidia добивается успеха с 4-битным
// форматом NVFP4", asector.ru, section "NVFP4 и Blackwell: интеграция
// архитектуры и формата"), a 16-element block multiplier that maps the block's
// largest magnitude to 6 ("Thinking Machines ускорила обучение Inkling 2 Small
// 4-битными числами", iitak.ru, section "Детали"), nearest-even and stochastic
// rounding (asector.ru page, same section; iitak.ru page, "Как это работает"),
// and the 16-point random Hadamard transform (asector.ru page, "Эксперименты и
// сравнение с FP8").
//
// Every helper is written for the VALU: integer tricks on binary32 bit
// patterns instead of searches or tables, no divisions on the per-element
// path (one correctly rounded division and one reciprocal per block), and
// the code is compiled with -ffp-contract=off so that each float operation
// rounds exactly once, as the format's definition requires.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies, the high halves
// XORed with the remaining counter words and the round key, the key advanced
// by the two Weyl increments after every round.
struct Words4 {
    uint32_t w[4];
};

__host__ __device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                         uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint64_t pa = (uint64_t)0xD2511F53u * c0;
        const uint64_t pb = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi_a = (uint32_t)(pa >> 32), lo_a = (uint32_t)pa;
        uint32_t hi_b = (uint32_t)(pb >> 32), lo_b = (uint32_t)pb;
        uint32_t n0 = hi_b ^ c1 ^ k0;
        uint32_t n2 = hi_a ^ c3 ^ k1;
        c0 = n0;
        c1 = lo_b;
        c2 = n2;
        c3 = lo_a;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Words4 r;
    r.w[0] = c0;
    r.w[1] = c1;
    r.w[2] = c2;
    r.w[3] = c3;
    return r;
}

// Random-stream identifiers (counter word 2).
enum : uint32_t { kStreamRow = 0, kStreamCol = 1, kStream2D = 2, kStreamHadamard = 3 };

// Hadamard sign mask: bits 0..15 of word 0 of Philox(key = seed, counter =
// (0, 0, 3, 0)); bit j set means sign -1 on element j of each 16-group.
__host__ __device__ inline uint32_t hadamard_sign_mask(uint64_t seed) {
    return philox4x32_10(0u, 0u, kStreamHadamard, 0u, (uint32_t)seed, (uint32_t)(seed >> 32)).w[0] &
           0xFFFFu;
}

// Device-side Philox rounds kept as a rolled loop (compact code, so that the
// callers' loops over blocks can be fully unrolled), advancing two counters
// that share a key in lockstep: two independent multiply chains per round.
__device__ __forceinline__ void philox4x32_10_pair(uint32_t a[4], uint32_t b[4], uint32_t k0,
                                                   uint32_t k1) {
#pragma unroll 1
    for (int i = 0; i < 10; ++i) {
        const uint64_t pa0 = (uint64_t)0xD2511F53u * a[0], pa1 = (uint64_t)0xCD9E8D57u * a[2];
        const uint64_t pb0 = (uint64_t)0xD2511F53u * b[0], pb1 = (uint64_t)0xCD9E8D57u * b[2];
        const uint32_t na0 = (uint32_t)(pa1 >> 32) ^ a[1] ^ k0, na2 = (uint32_t)(pa0 >> 32) ^ a[3] ^ k1;
        const uint32_t nb0 = (uint32_t)(pb1 >> 32) ^ b[1] ^ k0, nb2 = (uint32_t)(pb0 >> 32) ^ b[3] ^ k1;
        a[1] = (uint32_t)pa1;
        a[3] = (uint32_t)pa0;
        a[0] = na0;
        a[2] = na2;
        b[1] = (uint32_t)pb1;
        b[3] = (uint32_t)pb0;
        b[0] = nb0;
        b[2] = nb2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// Sixteen 16-bit draws for output elements base .. base+15 (base % 16 == 0):
// Philox with counters base/8 and base/8 + 1.  d[j] is the draw of element
// base + j (16 bits of word (j % 8) / 2, low half for even j).
__device__ __forceinline__ void draws16(uint64_t seed, uint32_t stream, uint64_t base,
                                        uint32_t d[16]) {
    const uint64_t q = base >> 3, q1 = q + 1;
    uint32_t a[4] = {(uint32_t)q, (uint32_t)(q >> 32), stream, 0u};
    uint32_t b[4] = {(uint32_t)q1, (uint32_t)(q1 >> 32), stream, 0u};
    philox4x32_10_pair(a, b, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        d[2 * j] = a[j] & 0xFFFFu;
        d[2 * j + 1] = a[j] >> 16;
        d[8 + 2 * j] = b[j] & 0xFFFFu;
        d[8 + 2 * j + 1] = b[j] >> 16;
    }
}

// Eight draws for each of two element groups (bases a_base and b_base, both
// multiples of 8): one paired Philox run.
__device__ __forceinline__ void draws8x2(uint64_t seed, uint32_t stream, uint64_t a_base,
                                         uint64_t b_base, uint32_t da[8], uint32_t db[8]) {
    const uint64_t qa = a_base >> 3, qb = b_base >> 3;
    uint32_t a[4] = {(uint32_t)qa, (uint32_t)(qa >> 32), stream, 0u};
    uint32_t b[4] = {(uint32_t)qb, (uint32_t)(qb >> 32), stream, 0u};
    philox4x32_10_pair(a, b, (uint32_t)seed, (uint32_t)(seed >> 32));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        da[2 * j] = a[j] & 0xFFFFu;
        da[2 * j + 1] = a[j] >> 16;
        db[2 * j] = b[j] & 0xFFFFu;
        db[2 * j + 1] = b[j] >> 16;
    }
}

// Eight draws for elements base .. base+7 (base % 8 == 0).
__device__ __forceinline__ void draws8(uint64_t seed, uint32_t stream, uint64_t base,
                                       uint32_t d[8]) {
    uint32_t unused[8];
    draws8x2(seed, stream, base, base + 8, d, unused);
}

// ---------------------------------------------------------------- formats
// binary32 value of an E4M3 byte (bias 7; exponent field 0 = multiples of 2^-9)
// (the gfx950 FP8 -> binary32 convert is exact for every finite E4M3 byte)
__device__ __forceinline__ float e4m3_value(uint32_t s) {
    return __builtin_amdgcn_cvt_f32_fp8((int)s, 0);
}

// Nearest E4M3 byte to u >= 0, ties to the even code, clamped to 448 (0x7E).
// The gfx950 FP8 convert rounds to nearest-even onto E4M3 (subnormals
// included) but does not saturate above 464; clamping to 448 first makes it
// the required clamp-then-round.
__device__ __forceinline__ uint32_t e4m3_encode(float u) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(fminf(u, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// E2M1 magnitude code (0..7) of y >= 0, round to nearest, ties to even,
// saturating at 6.  Below 1 the grid is the multiples of 0.5, so the code is
// rint(2y).  From 1 up, rounding the binary32 significand to one fraction bit
// (add 0x1FFFFF plus the kept bit, the classic nearest-even carry) lands on the
// grid and the kept (exponent, fraction-bit) pair is the code + 252.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
    uint32_t lo = (uint32_t)__builtin_rintf(y * 2.0f);
    uint32_t b = __float_as_uint(y);
    uint32_t r = b + 0x1FFFFFu + ((b >> 22) & 1u);
    uint32_t hi = min((r >> 22) - 252u, 7u);
    return y < 1.0f ? lo : hi;
}

// E2M1 magnitude code of y >= 0 by stochastic rounding with a 16-bit draw:
// round up iff r16 < f * 2^16, f the fraction of the way from the lower grid
// neighbour to the upper one.  From 1 up the neighbours differ in the first
// fraction bit, f * 2^16 = (low 22 fraction bits) / 64, so the test is the
// integer compare (r16 << 6) < low22.  Below 1 the grid step is 0.5 and
// f * 2^16 = y * 2^17 - (y >= 0.5) * 2^16; both sides of that compare are
// exact binary32 values.
__device__ __forceinline__ uint32_t e2m1_sr(float y, uint32_t r16) {
    uint32_t b = __float_as_uint(y);
    uint32_t up_hi = (r16 << 6) < (b & 0x3FFFFFu);
    uint32_t hi = min((b >> 22) - 252u + up_hi, 7u);
    uint32_t half = y >= 0.5f;
    float thr = (float)(r16 + (half << 16));
    uint32_t lo = half + (thr < y * 131072.0f);
    return y < 1.0f ? lo : hi;
}

// Per-tensor scale s_t = A_t / (6 * 448); 1 when that quotient is 0.
__device__ __forceinline__ float tensor_scale_of(float amax) {
    float st = amax / 2688.0f;
    return st > 0.0f ? st : 1.0f;
}

struct BlockScale {
    uint32_t byte;
    float R;
};

// Block multiplier: u = A_b / (6 s_t) rounded to E4M3; S = e4m3(u) * s_t;
// R = 1/S (0 when S is 0, which makes every magnitude 0).
__device__ __forceinline__ BlockScale block_scale(float amax_b, float six_st, float st) {
    BlockScale bs;
    float u = amax_b / six_st;
    bs.byte = e4m3_encode(u);
    float S = e4m3_value(bs.byte) * st;
    bs.R = S > 0.0f ? 1.0f / S : 0.0f;
    return bs;
}

// 4-bit codes of N values (N = 8 or 16; sign copied) packed into N/8 32-bit
// words, the even element in the low nibble.  d holds the 16-bit draws when
// SR is used.
//   RNE: the values are scaled first (y = t * R keeps the sign; its magnitude
//   is fl(|t| * R)), then the gfx950 FP4 pack instruction with scale operand
//   1.0 rounds two of them to nearest-even E2M1 with saturation at 6 and writes
//   their codes into one byte of the word.
//   SR: e2m1_sr on the magnitude, sign bit copied, nibbles packed in VALU.
template <bool SR, int N>
__device__ __forceinline__ void encode(const float* v, BlockScale bs, const uint32_t* d,
                                       uint32_t* out) {
    if (__builtin_expect(__builtin_isinf(bs.R), 0)) {
        // Reciprocal overflow (S below 2^-128): every nonzero element maps past
        // 6 and saturates; zeros stay zero.
#pragma unroll
        for (int k = 0; k < N / 8; ++k) out[k] = 0u;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            uint32_t c = (__float_as_uint(v[j]) >> 28) & 8u;
            c |= (v[j] != 0.0f) ? 7u : 0u;
            out[j >> 3] |= c << (4 * (j & 7));
        }
        return;
    }
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
        uint32_t w = 0u;
        if (!SR) {
            const float* p = v + 8 * k;
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[0] * bs.R, p[1] * bs.R, 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[2] * bs.R, p[3] * bs.R, 1.0f, 1);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[4] * bs.R, p[5] * bs.R, 1.0f, 2);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[6] * bs.R, p[7] * bs.R, 1.0f, 3);
        } else {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int j = 8 * k + jj;
                uint32_t bits = __float_as_uint(v[j]);
                float y = __uint_as_float(bits & 0x7FFFFFFFu) * bs.R;
                uint32_t mag = e2m1_sr(y, d[j]);
                w |= (((bits >> 28) & 8u) | mag) << (4 * jj);
            }
        }
        out[k] = w;
    }
}

// Two E2M1 codes (byte `sel` of w; low nibble first) as exact binary32 values,
// by the gfx950 FP4 unpack instruction with scale operand 1.0.
__device__ __forceinline__ float2 e2m1x2_unpack(uint32_t w, int sel) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    f2_t r;
    switch (sel) {
        case 0: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
        case 1: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
        case 2: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
        default: r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    return make_float2(r[0], r[1]);
}

// Two binary32 values -> packed bf16 pair (nearest-even), the first in the
// low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// E2M1 magnitude value (no sign) as binary32.
__device__ __forceinline__ float e2m1_value(uint32_t code) {
    uint32_t m = code & 7u;
    float mag = m < 2u ? 0.5f * (float)m : __uint_as_float(((m >> 1) + 126u) << 23 | (m & 1u) << 22);
    return (code & 8u) ? -mag : mag;
}

// ---------------------------------------------------------------- Hadamard
// t = (1/4) H16 D x: sign flips by mask bit, butterflies at distance 1, 2, 4, 8
// ((a, b) -> (a + b, a - b)), then the multiply by 1/4; binary32 throughout.
__device__ __forceinline__ void hadamard16(float v[16], uint32_t sign_mask) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if ((sign_mask >> j) & 1u) v[j] = -v[j];
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j & h) continue;
            float a = v[j], b = v[j + h];
            v[j] = a + b;
            v[j + h] = a - b;
        }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = 0.25f * v[j];
}

// ---------------------------------------------------------------- loads
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 8 consecutive bf16 elements (16 bytes, 16-byte aligned) -> binary32.
__device__ __forceinline__ void load8(const uint16_t* p, float v[8]) {
    uint4 q = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
}

// 8 consecutive binary32 elements (32 bytes, 16-byte aligned).
__device__ __forceinline__ void load8(const float* p, float v[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ float absmax16(const float v[16]) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
    return a;
}

}  // namespace nvfp4
