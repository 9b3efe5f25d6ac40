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

// Sixteen 16-bit draws for output elements base .. base+15 (base % 16 == 0):
// two Philox calls with counters base/8 and base/8 + 1.  d[j] is the draw of
// element base + j (16 bits of word (j % 8) / 2, low half for even j).
__device__ __forceinline__ void draws16(uint64_t seed, uint32_t stream, uint64_t base,
                                        uint32_t d[16]) {
    uint64_t q = base >> 3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint64_t qq = q + h;
        Words4 w = philox4x32_10((uint32_t)qq, (uint32_t)(qq >> 32), stream, 0u, (uint32_t)seed,
                                 (uint32_t)(seed >> 32));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            d[8 * h + 2 * j] = w.w[j] & 0xFFFFu;
            d[8 * h + 2 * j + 1] = w.w[j] >> 16;
        }
    }
}

// Eight draws for elements base .. base+7 (base % 8 == 0): one Philox call.
__device__ __forceinline__ void draws8(uint64_t seed, uint32_t stream, uint64_t base,
                                       uint32_t d[8]) {
    uint64_t q = base >> 3;
    Words4 w = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), stream, 0u, (uint32_t)seed,
                             (uint32_t)(seed >> 32));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        d[2 * j] = w.w[j] & 0xFFFFu;
        d[2 * j + 1] = w.w[j] >> 16;
    }
}

// ---------------------------------------------------------------- formats
// binary32 value of an E4M3 byte (bias 7; exponent field 0 = multiples of 2^-9).
__device__ __forceinline__ float e4m3_value(uint32_t s) {
    uint32_t e = s >> 3, m = s & 7u;
    return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

// Nearest E4M3 byte to u >= 0, ties to the even code, clamped to 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float u) {
    if (!(u > 0.0f)) return 0u;
    if (u >= 448.0f) return 0x7Eu;
    if (u < 0.015625f) return (uint32_t)__builtin_rintf(u * 512.0f);  // subnormal grid, 0..8
    uint32_t b = __float_as_uint(u);
    uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
    uint32_t rem = b & 0xFFFFFu;
    uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (code & 1u));
    return code + up;  // a carry out of the 3 mantissa bits bumps the exponent
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
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int j = 8 * k + jj;
            uint32_t bits = __float_as_uint(v[j]);
            float y = __uint_as_float(bits & 0x7FFFFFFFu) * bs.R;
            uint32_t mag = SR ? e2m1_sr(y, d[j]) : e2m1_rne(y);
            w |= (((bits >> 28) & 8u) | mag) << (4 * jj);
        }
        out[k] = w;
    }
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
