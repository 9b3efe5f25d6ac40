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

// Three-input XOR in one VALU instruction (gfx950 v_bitop3_b32, truth table
// 0x96); c is wave-uniform (a Philox round key).
__device__ __forceinline__ uint32_t xor3_vvs(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(c));
    return r;
}

// Device-side Philox: two counters that share a key advanced in lockstep
// (two independent multiply chains per round), fully unrolled, each round's
// two XORs fused into one instruction.  About 9.3 VALU instructions per round
// and counter.
__device__ __forceinline__ void philox4x32_10_pair(uint32_t a[4], uint32_t b[4], uint32_t k0,
                                                   uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint64_t pa0 = (uint64_t)0xD2511F53u * a[0], pa1 = (uint64_t)0xCD9E8D57u * a[2];
        const uint64_t pb0 = (uint64_t)0xD2511F53u * b[0], pb1 = (uint64_t)0xCD9E8D57u * b[2];
        const uint32_t na0 = xor3_vvs((uint32_t)(pa1 >> 32), a[1], k0);
        const uint32_t na2 = xor3_vvs((uint32_t)(pa0 >> 32), a[3], k1);
        const uint32_t nb0 = xor3_vvs((uint32_t)(pb1 >> 32), b[1], k0);
        const uint32_t nb2 = xor3_vvs((uint32_t)(pb0 >> 32), b[3], k1);
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

// Philox words of the 8-element groups that start at output indices a_base and
// b_base (multiples of 8): counters a_base/8 and b_base/8, one paired run.
// Word j of a group holds the 16-bit draws of elements 2j (low half) and
// 2j + 1 (high half).
__device__ __forceinline__ void philox_words2(uint64_t seed, uint32_t stream, uint64_t a_base,
                                              uint64_t b_base, uint32_t wa[4], uint32_t wb[4]) {
    const uint64_t qa = a_base >> 3, qb = b_base >> 3;
    wa[0] = (uint32_t)qa;
    wa[1] = (uint32_t)(qa >> 32);
    wa[2] = stream;
    wa[3] = 0u;
    wb[0] = (uint32_t)qb;
    wb[1] = (uint32_t)(qb >> 32);
    wb[2] = stream;
    wb[3] = 0u;
    philox4x32_10_pair(wa, wb, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Words of the 16 elements base .. base+15 (base % 16 == 0): w[0..3] for the
// first 8, w[4..7] for the second 8.
__device__ __forceinline__ void philox_words16(uint64_t seed, uint32_t stream, uint64_t base,
                                               uint32_t w[8]) {
    philox_words2(seed, stream, base, base + 8, w, w + 4);
}

// Words of the 8 elements base .. base+7 (base % 8 == 0).
__device__ __forceinline__ void philox_words8(uint64_t seed, uint32_t stream, uint64_t base,
                                              uint32_t w[4]) {
    uint32_t unused[4];
    philox_words2(seed, stream, base, base + 8, w, unused);
}

// 16-bit draw of element j of a group (word j / 2, low half for even j).
__device__ __forceinline__ uint32_t draw16(const uint32_t* w, int j) {
    return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
}

// ---------------------------------------------------------------- lane exchanges
// Exchanges inside aligned groups of four lanes as DPP quad permutes: the
// value of another lane of the quad arrives as a VALU operand modifier
// instead of through an LDS round trip (ds_bpermute).  Control word: output
// lane i of each quad reads input lane (CTRL >> 2i) & 3.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_perm(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
    return __uint_as_float(quad_perm<CTRL>(__float_as_uint(x)));
}
// The value of lane ^ 1 and of lane ^ 2.
template <typename V>
__device__ __forceinline__ V lane_xor1(V x) { return quad_perm<0xB1>(x); }
template <typename V>
__device__ __forceinline__ V lane_xor2(V x) { return quad_perm<0x4E>(x); }
// The value of lane k of the caller's aligned group of G (2 or 4) lanes.
template <int G, typename V>
__device__ __forceinline__ V group_lane(V x, int k) {
    if constexpr (G == 2) {
        return k == 0 ? quad_perm<0xA0>(x) : quad_perm<0xF5>(x);  // [0,0,2,2], [1,1,3,3]
    } else {
        return k == 0 ? quad_perm<0x00>(x) : k == 1 ? quad_perm<0x55>(x)
             : k == 2 ? quad_perm<0xAA>(x) : quad_perm<0xFF>(x);  // [k,k,k,k]
    }
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

// Multiplier of E4M3 byte b for a tensor with scale s_t: S = e4m3(b) * s_t,
// R = 1/S (0 when S is 0, which makes every magnitude 0).  A block's S is one
// of the 127 values S(b), so a workgroup computes R(b) once per byte into a
// table (the same binary32 operations) and blocks look it up instead of
// dividing.  Byte 0x7F (NaN) gives 0 and is never produced by e4m3_encode.
__device__ __forceinline__ float block_multiplier(uint32_t b, float st) {
    const float S = e4m3_value(b) * st;
    return S > 0.0f ? 1.0f / S : 0.0f;
}

// Block scale: u = A_b / (6 s_t) rounded to E4M3 (the byte), R from the
// tensor's multiplier table rtab[128].
__device__ __forceinline__ BlockScale block_scale(float amax_b, float six_st, const float* rtab) {
    BlockScale bs;
    bs.byte = e4m3_encode(amax_b / six_st);
    bs.R = rtab[bs.byte];
    return bs;
}

// Seed operand of the gfx950 stochastic-rounding FP4 convert for a 16-bit
// draw r16.  That instruction adds the top 22 bits of its seed to the 22
// binary32 significand bits below the kept E2M1 bit and truncates.  With seed
// = ~(r16 << 16) those 22 bits are (65535 - r16) * 64 + 63, so the carry
// happens exactly when F > 64 r16, F the 22 fraction bits: round up iff
// r16 < f * 2^16 whenever the whole fraction f fits in those 22 bits.  For
// inputs below 1 the instruction first shifts the significand right and drops
// the bits shifted out; feeding it the value rounded up to a multiple of
// 2^-23 makes the dropped bits zero, and since r16 * 64 is an integer,
// "64 r16 < ceil(f 2^22)" is the same decision as "64 r16 < f 2^22".  (This
// pairing of seed and pre-rounding was checked against the integer rule of
// e2m1_sr over 3.6e8 value/draw pairs spanning every E2M1 interval, binary32
// subnormals and both signs, for the instruction's first slot; its second
// slot does not follow this rule, so every call here converts one value, in
// the first slot.)
__device__ __forceinline__ uint32_t sr_seed(uint32_t word, int high_half) {
    const uint32_t nw = ~word;
    return high_half ? (nw | 0xFFFFu) : ((nw << 16) | 0xFFFFu);
}

// 4-bit codes of N values (N = 8 or 16; sign copied) packed into N/8 32-bit
// words, the even element in the low nibble.  w holds the Philox words of the
// N elements (draws of elements 2j, 2j+1 in word j) when SR is used; amax_b
// is the block's largest magnitude.
//   RNE: the values are scaled first (y = t * R keeps the sign; its magnitude
//   is fl(|t| * R)), then the gfx950 FP4 pack instruction with scale operand
//   1.0 rounds two of them to nearest-even E2M1 with saturation at 6 and writes
//   their codes into one byte of the word.
//   SR: y = fl(|t| * R), z = ceil(y * 2^23) carries t's sign, and the SR
//   convert with scale operand 2^23 (so it sees z * 2^-23, y rounded up to the
//   2^-23 grid) and seed sr_seed(draw) produces the code.  Each call converts
//   one value in the instruction's first slot into the low nibble of byte 0
//   of a fresh register (the second slot's input is left unspecified and the
//   rest of the register is masked off; the compiler does not carry the
//   builtin's `old` operand through); byte permutes then gather the codes of
//   even and odd elements into the low and high nibbles of the output word.
//   Blocks with R = inf (S below 2^-128), or whose scaled values could
//   overflow (amax_b * R >= 2^100, possible only with a caller-supplied A_t
//   below the true one), take the plain VALU path of e2m1_rne / e2m1_sr.
// Codes of the 8 values p[0..7] by stochastic rounding into one word (see
// encode).  FOLD computes z = ceil(fl(|t| * R23)) with R23 = R * 2^23, one
// multiply instead of two; the caller guarantees that this equals
// ceil(fl(|t| * R) * 2^23).
typedef float sr_f2_t __attribute__((ext_vector_type(2)));

// The SR FP4 convert writing only byte SEL of acc (its op_sel bits 2 and 3
// select the destination byte; the other three bytes keep their value, and
// SEL 0, written first, takes none in).
// Written as asm with acc tied in and out: the compiler's builtin for this
// instruction treats the whole destination register as written.
template <int SEL>
__device__ __forceinline__ void cvt_sr_fp4_byte(uint32_t& acc, sr_f2_t v, uint32_t seed, float scale) {
    if constexpr (SEL == 0)  // (the first of a word's four: the other bytes are written later)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "=v"(acc) : "v"(v), "v"(seed), "s"(scale));
    else if constexpr (SEL == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(acc) : "v"(v), "v"(seed), "s"(scale));
    else if constexpr (SEL == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(acc) : "v"(v), "v"(seed), "s"(scale));
    else
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(acc) : "v"(v), "v"(seed), "s"(scale));
}

template <bool FOLD>
__device__ __forceinline__ uint32_t sr_word8(const float* p, float R, const uint32_t* wk) {
    const float R23 = R * 0x1p23f;
    // byte J of ev / od: code of element 2J / 2J + 1 in the low nibble (the
    // high nibble, from the unspecified second slot, is masked off); every
    // byte is written, byte 0 first
    uint32_t ev, od;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        const float z0 = FOLD ? __builtin_ceilf(fabsf(p[2 * J]) * R23)
                              : __builtin_ceilf((fabsf(p[2 * J]) * R) * 0x1p23f);
        const float z1 = FOLD ? __builtin_ceilf(fabsf(p[2 * J + 1]) * R23)
                              : __builtin_ceilf((fabsf(p[2 * J + 1]) * R) * 0x1p23f);
        const float any = __builtin_nondeterministic_value(z0);
        const sr_f2_t e = {__uint_as_float(__float_as_uint(z0) | (__float_as_uint(p[2 * J]) & 0x80000000u)), any};
        const sr_f2_t o = {__uint_as_float(__float_as_uint(z1) | (__float_as_uint(p[2 * J + 1]) & 0x80000000u)), any};
        switch (J) {
            case 0: cvt_sr_fp4_byte<0>(ev, e, sr_seed(wk[J], 0), 0x1p23f); cvt_sr_fp4_byte<0>(od, o, sr_seed(wk[J], 1), 0x1p23f); break;
            case 1: cvt_sr_fp4_byte<1>(ev, e, sr_seed(wk[J], 0), 0x1p23f); cvt_sr_fp4_byte<1>(od, o, sr_seed(wk[J], 1), 0x1p23f); break;
            case 2: cvt_sr_fp4_byte<2>(ev, e, sr_seed(wk[J], 0), 0x1p23f); cvt_sr_fp4_byte<2>(od, o, sr_seed(wk[J], 1), 0x1p23f); break;
            default: cvt_sr_fp4_byte<3>(ev, e, sr_seed(wk[J], 0), 0x1p23f); cvt_sr_fp4_byte<3>(od, o, sr_seed(wk[J], 1), 0x1p23f); break;
        }
    }
    return (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
}

template <bool SR, int N, bool FOLD = false>
__device__ __forceinline__ void encode(const float* v, BlockScale bs, float amax_b, const uint32_t* w,
                                       uint32_t* out) {
    const bool slow = SR ? !(amax_b * bs.R < 0x1p100f) : __builtin_isinf(bs.R);
    if (__builtin_expect(slow, 0)) {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) out[k] = 0u;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const uint32_t bits = __float_as_uint(v[j]);
            const float a = __uint_as_float(bits & 0x7FFFFFFFu);
            const float y = a == 0.0f ? 0.0f : a * bs.R;  // (0 * inf would be NaN)
            const uint32_t mag = SR ? e2m1_sr(y, draw16(w, j)) : e2m1_rne(y);
            out[j >> 3] |= (((bits >> 28) & 8u) | mag) << (4 * (j & 7));
        }
        return;
    }
    if (!SR) {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) {
            const float* p = v + 8 * k;
            uint32_t c = 0u;
            c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, p[0] * bs.R, p[1] * bs.R, 1.0f, 0);
            c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, p[2] * bs.R, p[3] * bs.R, 1.0f, 1);
            c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, p[4] * bs.R, p[5] * bs.R, 1.0f, 2);
            c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, p[6] * bs.R, p[7] * bs.R, 1.0f, 3);
            out[k] = c;
        }
        return;
    }
    // FOLD (BF16 inputs, no transform): every nonzero |t| is at least 2^-133.
    // With R = 0 or 2^-16 <= R < 2^100, fl(|t| * R) is 0 only for t = 0; when
    // it is normal, scaling by 2^23 commutes with the rounding, and when it is
    // subnormal both forms give z = 1.  So the single multiply by R * 2^23 gives
    // the same z.  The wave takes that path when every active lane qualifies.
    if (FOLD && __all(bs.R == 0.0f || (bs.R >= 0x1p-16f && bs.R < 0x1p100f))) {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) out[k] = sr_word8<true>(v + 8 * k, bs.R, w + 4 * k);
    } else {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) out[k] = sr_word8<false>(v + 8 * k, bs.R, w + 4 * k);
    }
}

// encode<SR, 16> of t = h / 4 given h, the 16 sums of hadamard16_sums over
// sign-flipped BF16 inputs (amax_b is the block's largest |t|).  Every such h
// is a multiple of 2^-133, so t = h / 4 is exact (binary32 subnormals are
// multiples of 2^-149), and whenever R / 4 is exact, fl(|t| R) = fl(|h| (R / 4)):
// the multiply by 1/4 folds into the block multiplier.  With SR the single
// multiply by R / 4 * 2^23 of the FOLD path then holds too (as there, with
// nonzero |h| >= 2^-133 it needs R / 4 >= 2^-16).  A wave whose lanes do not
// all qualify forms t and takes the general path.
template <bool SR>
__device__ __forceinline__ void encode_quarter16(float h[16], BlockScale bs, float amax_b, const uint32_t* w,
                                                 uint32_t* out) {
    const bool slow = SR ? !(amax_b * bs.R < 0x1p100f) : __builtin_isinf(bs.R);
    if (SR) {
        if (__all(!slow && (bs.R == 0.0f || (bs.R >= 0x1p-14f && bs.R < 0x1p100f)))) {
            const float Rq = 0.25f * bs.R;
            out[0] = sr_word8<true>(h, Rq, w);
            out[1] = sr_word8<true>(h + 8, Rq, w + 4);
            return;
        }
    } else {
        if (__all(!slow && (bs.R == 0.0f || bs.R >= 0x1p-124f))) {
            BlockScale q = bs;
            q.R = 0.25f * bs.R;
            encode<false, 16>(h, q, amax_b, w, out);
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) h[j] = 0.25f * h[j];
    encode<SR, 16, false>(h, bs, amax_b, w, out);
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

// The butterflies of hadamard16 alone (no sign flips, no multiply by 1/4), in
// the same order: h = H16 x.
__device__ __forceinline__ void hadamard16_sums(float v[16]) {
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
}

// max_i |t_i| of t = hadamard16(v): the same values as transforming and then
// taking the maximum magnitude, with less work.  For binary32 a and b, one of
// |a + b| and |a - b| is |a| + |b| exactly and the other is smaller, and
// rounding is monotone and sign-symmetric, so max(|fl(a + b)|, |fl(a - b)|) =
// fl(|a| + |b|): the last butterfly stage collapses to one addition per pair.
// fl(x / 4) is monotone in |x| too, so the multiply by 1/4 moves after the
// maximum.
__device__ __forceinline__ float hadamard16_absmax(float v[16], uint32_t sign_mask) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
        if ((sign_mask >> j) & 1u) v[j] = -v[j];
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j & h) continue;
            float a = v[j], b = v[j + h];
            v[j] = a + b;
            v[j + h] = a - b;
        }
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]) + fabsf(v[j + 8]));
    return 0.25f * m;
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

// ---------------------------------------------------------------- tiles
// Tile of the calling workgroup.  Workgroups are handed to the eight XCDs
// round robin in dispatch order, and each XCD has its own L2.  With
// xcd_group = G (> 1; G divides the grid width), each run of G consecutive
// tiles along a tile row is served by workgroups of one XCD: within every
// block of 8 G dispatched workgroups, workgroup L takes tile
// G * (L % 8) + (L / 8) % G of the block.  Output lines that those G tiles
// write in parts (row codes and scales of the fused layout) are then
// completed in one L2, and the G tiles' row segments are read by one L2 as
// one contiguous stretch.  A last partial block keeps the identity order.
struct TileXY {
    int64_t x, y;
};

__device__ __forceinline__ TileXY xcd_tile(int xcd_group) {
    const int64_t gx = gridDim.x;
    int64_t L = (int64_t)blockIdx.y * gx + blockIdx.x;
    if (xcd_group > 1) {
        const int64_t blk = 8 * (int64_t)xcd_group;
        if (L < ((int64_t)gridDim.y * gx) / blk * blk)
            L = L / blk * blk + xcd_group * (L % 8) + (L / 8) % xcd_group;
    }
    TileXY r;
    r.x = L % gx;
    r.y = L / gx;
    return r;
}

// As xcd_tile, but each XCD's run of xcd_group tiles covers xcd_group / 2
// tiles along x on each of two consecutive tile rows (when the grid width is a
// multiple of 4 xcd_group; a last odd tile row then keeps the dispatch order,
// and other widths take the xcd_tile order).  Column-blocked outputs write 16 scale bytes per column
// and tile, half of a 32-byte sector whose other half belongs to the tile
// below: pairing the two rows on one XCD lets its L2 join the halves, where
// runs along one row left them to two L2s.
__device__ __forceinline__ TileXY xcd_tile_pairs(int xcd_group) {
    const int64_t gx = gridDim.x, gy = gridDim.y;
    const int64_t L = (int64_t)blockIdx.y * gx + blockIdx.x;
    if (xcd_group > 1 && xcd_group % 2 == 0 && gx % (4 * xcd_group) == 0 && L < (gy / 2) * 2 * gx) {
        const int64_t H = xcd_group / 2, blk = 8 * (int64_t)xcd_group;
        const int64_t b = L / blk, w = L % blk;
        const int64_t k = w % 8, j = w / 8;
        const int64_t bpr = gx / (8 * H);  // blocks per pair of tile rows
        TileXY r;
        r.x = (b % bpr) * 8 * H + k * H + j % H;
        r.y = (b / bpr) * 2 + j / H;
        return r;
    }
    if (xcd_group > 1 && xcd_group % 2 == 0 && gx % (4 * xcd_group) == 0) {
        TileXY r;
        r.x = L % gx;
        r.y = L / gx;
        return r;
    }
    return xcd_tile(xcd_group);
}

// ------------------------------------------------------------ GEMM tile stores
// Store a wave's block of I x J 32x32 MFMA accumulator tiles, scaled by
// value(i, j, r) (accumulator r of tile (i, j): row 32 i + 8 (r / 4) + 4 h +
// r % 4, column 32 j + l32 of the block), when the whole block -- 32 I rows
// from row0 and 32 J columns from col0 -- lies inside C (the caller checks)
// and 32 I rows of C span under 2^31 bytes (checked here: false is returned
// and nothing is stored otherwise).  The stores go through a buffer resource
// based at the block's first element: each lane at a fixed byte offset, each
// row's offset in a scalar register, each 32-column block in the
// instruction's immediate offset, rows converted to BF16 in pairs.  Written
// the plain way, an element costs 64-bit address arithmetic, a bounds compare
// and a branch around its store.
typedef float gemm_f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 gemm_bf2_t __attribute__((ext_vector_type(2)));

template <int I, int J, bool OUT_BF16, typename Value>
__device__ __forceinline__ bool store_wave_block(void* C, int64_t ldc, int64_t row0, int64_t col0, int h, int l32,
                                                 Value value) {
    constexpr int ES = OUT_BF16 ? 2 : 4;
    if (ldc > (int64_t)(INT32_MAX / (32 * I * ES))) return false;
    const int64_t bytes = ((32 * I - 1) * ldc + 32 * J) * ES;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char*>(C) + (row0 * ldc + col0) * ES, (short)0, (int)(uint32_t)bytes, 0x00020000);
    const int ldb = (int)ldc * ES, vo = 4 * h * ldb + ES * l32;
#pragma unroll
    for (int i = 0; i < I; ++i)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int so = (32 * i + 8 * (r >> 2) + (r & 3)) * ldb;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const float v0 = value(i, j, r), v1 = value(i, j, r + 1);
                if (OUT_BF16) {
                    const gemm_f2_t x = {v0, v1};
                    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, gemm_bf2_t));
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b, rc, vo + 32 * ES * j, so, 0);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(b >> 16), rc, vo + 32 * ES * j, so + ldb, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v0), rc, vo + 32 * ES * j, so, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v1), rc, vo + 32 * ES * j, so + ldb, 0);
                }
            }
        }
    return true;
}

}  // namespace nvfp4
