// device.h -- gfx950 device helpers for block-scaled FP4 quantization.
//
// Element encoders work on 8 elements at a time and return one packed dword
// (element j in nibble j), the unit the kernels store.  E2M1 rounding uses
// the gfx950 scaled-convert instructions:
//   v_cvt_scalef32_pk_fp4_f32     round to nearest even, saturating at 6
//   v_cvt_scalef32_sr_pk_fp4_f32  with a zero random word: truncation, i.e.
//                                 the lower bracketing codeword; with a word
//                                 built from the random byte: stochastic
//                                 rounding, exact for values with at most 14
//                                 significant bits (MXFP4 without the RHT) and
//                                 for multiples of 2^-23 (every other value is
//                                 first rounded up in magnitude to one)
// with a power-of-two scale (1.0, 2^e or 2^23) that the instruction divides
// by exactly.  The uniform grid is computed with plain fp32/integer
// arithmetic.  Per-block work (scale codes and reciprocals) is written in
// ordinary IEEE fp32 (correctly rounded division, denormals kept).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Streaming memory access.  Inputs are read once: non-temporal loads keep them
// from displacing reusable lines.  Quantize outputs take non-temporal stores when
// the caller says they are not read again soon (fp4_cfg.stream_out); the other
// outputs when FP4Q_NT_STORES is set (default off).
#ifndef FP4Q_NT_STORES
#define FP4Q_NT_STORES 0
#endif

#ifndef FP4Q_NT_LOADS
#define FP4Q_NT_LOADS 1
#endif

__device__ __forceinline__ void load16_nt(const uint16_t* p, uint32_t w[4]) {
    const v4u32* s = reinterpret_cast<const v4u32*>(p);
    const v4u32 a = FP4Q_NT_LOADS ? __builtin_nontemporal_load(s) : s[0];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
}

// nt: a non-temporal store (the caller's output is not read again soon).
template <typename T>
__device__ __forceinline__ void st_out(T* p, T v, bool nt = FP4Q_NT_STORES) {
    if (nt) __builtin_nontemporal_store(v, p);
    else *p = v;
}

__device__ __forceinline__ void st_out2(void* base, uint32_t idx, uint32_t a, uint32_t b, bool nt = FP4Q_NT_STORES) {
    v2u32 v = {a, b};
    st_out(reinterpret_cast<v2u32*>(base) + idx, v, nt);
}

__device__ __forceinline__ void st_out4(void* base, int64_t idx, uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                        bool nt = FP4Q_NT_STORES) {
    v4u32 v = {a, b, c, d};
    st_out(reinterpret_cast<v4u32*>(base) + idx, v, nt);
}

// Non-temporal 16-byte store, for an output several times larger than its
// input that streams out (a dequantized tensor): measured with the five-kernel
// 16384 x 4096 MXFP4 step, dequantizing with these stores made the whole step
// 7% faster (127 -> 118 us), since the 128 MiB of bf16 no longer evict the codes
// and guides the next kernels read; for the quantize kernels, whose outputs the
// next kernel reads, non-temporal stores made the step 3% slower.
__device__ __forceinline__ void st_stream4(void* base, int64_t idx, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    __builtin_nontemporal_store((v4u32){a, b, c, d}, reinterpret_cast<v4u32*>(base) + idx);
}

constexpr float kFltMax = 3.40282346638528859812e+38f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- E4M3 / E8M0

// E4M3FN code of t in [0, 448] (callers clamp), round to nearest even: the gfx950
// fp8 convert (OCP E4M3FN, bias 7, subnormal step 2^-9), one instruction.  It
// equals the rounding rule on every fp32 value in [0, 448] (checked on the GPU
// over all of them through fp4_encode_scales).  The second converted value is 0,
// so byte 1 of the result is 0 and the code needs no mask.
__device__ __forceinline__ uint32_t e4m3_encode_rne(float t) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false);
}

// min(t, 448) for t >= 0 or NaN, on the bit patterns (a NaN gives 448).
__device__ __forceinline__ float clamp448(float t) {
    return __uint_as_float(min(__float_as_uint(t), 0x43E00000u));
}

// Exact fp32 value of an E4M3FN magnitude code (sign bit ignored, 0x7F not special).
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
    code &= 0x7Fu;
    uint32_t e = code >> 3;
    float sub = (float)(code & 7u) * 0.001953125f;   // m * 2^-9
    float nrm = __uint_as_float((code << 20) + (120u << 23));
    return e == 0 ? sub : nrm;
}

// NVFP4 block reciprocal from a scale code: inv = RN(1/RN(dec*s_t)), 0 when the
// product is 0, FLT_MAX when the reciprocal overflows.
__device__ __forceinline__ float nvfp4_inv(uint32_t code, float ts) {
    float S = e4m3_decode(code) * ts;
    float inv = 1.0f / S;
    inv = __builtin_isinf(inv) ? kFltMax : inv;
    return S == 0.0f ? 0.0f : inv;
}

// MXFP4: 2^-e from the E8M0 code (code = e + 127, 0..254); code 254 gives the
// subnormal 2^-127.
__device__ __forceinline__ float mx_inv(uint32_t code) {
    return __uint_as_float(code < 254u ? (254u - code) << 23 : 0x00400000u);
}

// MXFP4: 2^e from the E8M0 code (code 0 gives the subnormal 2^-127).
__device__ __forceinline__ float mx_scale(uint32_t code) {
    return __uint_as_float(code ? code << 23 : 0x00400000u);
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon et al., SC'11: ten rounds of two 32x32->64 products with the published
// multipliers, Weyl-sequence key schedule.
struct u32x4 { uint32_t w[4]; };

// a ^ b ^ c in one instruction (truth table 0x96 = odd parity of the three bits)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                               uint32_t key0, uint32_t key1) {
    #pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t a = (uint64_t)x0 * 0xD2511F53u;
        const uint64_t b = (uint64_t)x2 * 0xCD9E8D57u;
        const uint32_t y0 = xor3((uint32_t)(b >> 32), x1, key0);
        const uint32_t y2 = xor3((uint32_t)(a >> 32), x3, key1);
        x1 = (uint32_t)b;
        x3 = (uint32_t)a;
        x0 = y0;
        x2 = y2;
        key0 += 0x9E3779B9u;
        key1 += 0xBB67AE85u;
    }
    u32x4 r;
    r.w[0] = x0; r.w[1] = x1; r.w[2] = x2; r.w[3] = x3;
    return r;
}

// ---------------------------------------------------------------- bit helpers

// 8 bits -> bit 4j of a dword (nibble LSBs).
__device__ __forceinline__ uint32_t spread8_to_nibbles(uint32_t b) {
    b &= 0xFFu;
    b = (b | (b << 12)) & 0x000F000Fu;
    b = (b | (b << 6)) & 0x03030303u;
    b = (b | (b << 3)) & 0x11111111u;
    return b;
}

// bit 4j of a dword -> 8 contiguous bits.
__device__ __forceinline__ uint32_t gather_nibble_lsbs(uint32_t w) {
    uint32_t x = w & 0x11111111u;
    x = (x | (x >> 3)) & 0x03030303u;
    x = (x | (x >> 6)) & 0x000F000Fu;
    x = (x | (x >> 12)) & 0xFFu;
    return x;
}

// ---------------------------------------------------------------- E2M1 converts

// The converts divide their inputs by the scale operand; with a power of two
// the result equals converting the exactly scaled value (checked on the GPU for
// every finite bf16 input, scales 2^-127..2^127, RNE and every SR word used here).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_rne2(uint32_t old, float a, float b, float scale = 1.0f) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

__device__ __forceinline__ uint32_t pack_rne8(const float v[8], float scale = 1.0f) {
    uint32_t w = 0;
    w = cvt_rne2<0>(w, v[0], v[1], scale);
    w = cvt_rne2<1>(w, v[2], v[3], scale);
    w = cvt_rne2<2>(w, v[4], v[5], scale);
    w = cvt_rne2<3>(w, v[6], v[7], scale);
    return w;
}

// RNE of 8 bf16 values (4 dwords, element 2j in the low half of w[j]) divided
// by a power-of-two scale, straight from the bf16 bits: the bf16-input convert
// equals the fp32-input one on every finite bf16 value (checked on the GPU for
// scales 2^-127..2^127) and also merges into the old destination bytes.
__device__ __forceinline__ uint32_t pack_rne8_bf16(const uint32_t w[4], float scale) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[0]), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[1]), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[2]), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, w[3]), scale, 3);
    return r;
}

// Byte 0 of four convert results -> one dword (two byte permutes and an or).
__device__ __forceinline__ uint32_t gather_b0(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3) {
    return __builtin_amdgcn_perm(r1, r0, 0x0C0C0400u) | __builtin_amdgcn_perm(r3, r2, 0x04000C0Cu);
}

__device__ __forceinline__ uint32_t pack_trunc8(const float v[8]) {
    uint32_t r[4];
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        v2f x = {v[2 * j], v[2 * j + 1]};
        r[j] = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, x, 0u, 1.0f, 0);
    }
    return gather_b0(r[0], r[1], r[2], r[3]);
}

// Truncation of 8 bf16 values (4 dwords) divided by a power-of-two scale,
// straight from the bf16 bits: equal to the fp32-input truncation on every
// bf16 bit pattern (checked on the GPU, both slots, scales 2^-127..2^127).
__device__ __forceinline__ uint32_t pack_trunc8_bf16(const uint32_t w[4], float scale) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    uint32_t r[4];
    #pragma unroll
    for (int j = 0; j < 4; ++j)
        r[j] = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_bf16(0u, __builtin_bit_cast(bf16x2_t, w[j]), 0u, scale, 0);
    return gather_b0(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ uint32_t sign_nibble(float v) { return (__float_as_uint(v) >> 28) & 8u; }

// ---------------------------------------------------------------- encoders
// v[j]: signed scaled values RN(y_j * inv).  Grid 0 = E2M1, 1 = uniform.

enum { MODE_RTN = 0, MODE_SR = 1, MODE_GUIDED = 2 };

// Guided E2M1 from L = truncation codes (lower bracket member, with sign) and
// Ld = truncation codes of the next smaller magnitude of each value.  A value
// lies on a codeword exactly when L and Ld differ (for +-0 the next smaller
// magnitude is a NaN pattern, which converts to a saturated code, also
// different), or when L has magnitude 7: every value at or above 6 saturates
// there and clamps to the codeword 6.  Off the grid the upper member is L+1
// (never carries into the sign: the magnitude is at most 6 there); it is taken
// when the LSB of L differs from the guide bit.
__device__ __forceinline__ uint32_t guided_from_trunc(uint32_t L, uint32_t Ld, uint32_t gbits) {
    uint32_t d = L ^ Ld;
    d |= d >> 1;
    d |= d >> 2;
    const uint32_t seven = (((L & 0x77777777u) + 0x11111111u) & 0x88888888u) >> 3;
    const uint32_t on_grid = (d | seven) & 0x11111111u;
    const uint32_t mism = (L ^ spread8_to_nibbles(gbits)) & 0x11111111u;
    return L + (mism & ~on_grid);
}

// v: already scaled values; the next smaller magnitude is the fp32 bit
// pattern minus one.
__device__ __forceinline__ uint32_t encode8_guided_e2m1(const float v[8], uint32_t gbits) {
    float vd[8];
    #pragma unroll
    for (int j = 0; j < 8; ++j) vd[j] = __uint_as_float(__float_as_uint(v[j]) - 1u);
    return guided_from_trunc(pack_trunc8(v), pack_trunc8(vd), gbits);
}

// MXFP4 without the RHT: w are the bf16 inputs, the convert divides by
// scale = 2^e.  The next smaller bf16 magnitude (pattern minus one per half)
// serves as well as the next smaller fp32 one: every codeword times 2^e is a
// bf16 value, so no codeword lies strictly between the two.
__device__ __forceinline__ uint32_t encode8_guided_e2m1_bf16(const uint32_t w[4], uint32_t gbits, float scale) {
    uint32_t wd[4];
    #pragma unroll
    for (int j = 0; j < 4; ++j)
        wd[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w[j]) - (u16x2){1, 1});
    return guided_from_trunc(pack_trunc8_bf16(w, scale), pack_trunc8_bf16(wd, scale), gbits);
}

// SR E2M1: the grid is uniform with step 0.5, 1, 2 on [0,2), [2,4), [4,6], and
// an element rounds up iff the fraction f of its bracket exceeds c = (2u+1)/512,
// i.e. iff |v| > lo + c * step.  Every such threshold, and every bracket end, is a
// multiple of 2^-10.
//
// The hardware convert, one element per instruction (slot 0; slot 1 converts
// +0), rounds up iff D + R >= 2^32, with D the discarded fraction of the bracket
// as a 32-bit fixed-point number; the word R = (~u << 24) | 0x7FFFFF makes that
// "D > (2u+1) * 2^23", i.e. 2u+1 < 512 f.  It is exact except below 1.0, where it
// keeps 23 fraction bits of v.  Checked on the GPU against the rule above over
// every fp32 value in [-8, 8] and every u: the only differences are values lying
// strictly within 2^-23 above a threshold, which have 15 or more significant
// bits.  So it is exact for every multiple of 2^-23 (encode8_sr_e2m1_w below),
// and for every value with at most 14 significant bits (MXFP4 without the RHT
// scales bf16 inputs by a power of two, so its v has at most 8).
// nw = ~(four random bytes); byte j of nw becomes the top byte of R.
__device__ __forceinline__ uint32_t sr_word(uint32_t nw, int j) {
    return __builtin_amdgcn_perm(nw, 0x007FFFFFu, ((4u + (uint32_t)j) << 24) | 0x020100u);
}

// The SR convert of the pair p, written into byte SEL of acc (slot 0's code in
// the byte's low nibble, slot 1's in its high nibble).  The instruction keeps
// the other three bytes of its destination (checked on the GPU for every byte
// position), but the builtin does not model that merge, so the destination is
// tied here in asm.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_sr_byte(uint32_t acc, v2f p, uint32_t R, float scale) {
    if constexpr (SEL == 0) asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(acc) : "v"(p), "v"(R), "v"(scale));
    if constexpr (SEL == 1)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(acc) : "v"(p), "v"(R), "v"(scale));
    if constexpr (SEL == 2)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(acc) : "v"(p), "v"(R), "v"(scale));
    if constexpr (SEL == 3)
        asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(acc) : "v"(p), "v"(R), "v"(scale));
    return acc;
}

// Slot 1 of the convert uses its random word shifted left by one, so each pair
// (v[2i], v[2i+1]) is converted twice from one register pair: with R for
// element 2i, whose code lands in the low nibble of byte i of e, and with
// R' >> 1 for element 2i+1, whose code lands in the high nibble of byte i of o
// (bit 0 of R' is below the convert's resolution; same exhaustive check as
// slot 0).  The other nibbles hold the other slot's code and are masked off.
__device__ __forceinline__ uint32_t encode8_sr_e2m1_short(const float v[8], uint32_t rnd0, uint32_t rnd1,
                                                          float scale = 1.0f) {
    const uint32_t n0 = ~rnd0, n1 = ~rnd1;
    uint32_t e = 0u, o = 0u;
    e = cvt_sr_byte<0>(e, (v2f){v[0], v[1]}, sr_word(n0, 0), scale);
    o = cvt_sr_byte<0>(o, (v2f){v[0], v[1]}, sr_word(n0, 1) >> 1, scale);
    e = cvt_sr_byte<1>(e, (v2f){v[2], v[3]}, sr_word(n0, 2), scale);
    o = cvt_sr_byte<1>(o, (v2f){v[2], v[3]}, sr_word(n0, 3) >> 1, scale);
    e = cvt_sr_byte<2>(e, (v2f){v[4], v[5]}, sr_word(n1, 0), scale);
    o = cvt_sr_byte<2>(o, (v2f){v[4], v[5]}, sr_word(n1, 1) >> 1, scale);
    e = cvt_sr_byte<3>(e, (v2f){v[6], v[7]}, sr_word(n1, 2), scale);
    o = cvt_sr_byte<3>(o, (v2f){v[6], v[7]}, sr_word(n1, 3) >> 1, scale);
    return (e & 0x0F0F0F0Fu) | (o & 0xF0F0F0F0u);
}

// SR E2M1 of values with any number of significant bits, given as w = 2^23 v.
// |w| is rounded up to an integer (sign kept): no threshold or bracket end
// lies strictly between |v| and that integer times 2^-23, so SR rounds both the
// same way, and the convert is exact for the latter.  The convert then divides
// by the scale 2^23 itself: for every integer-valued c up to 2^26 this equals
// converting c * 2^-23, and every |c| of 2^26 or more, infinity included,
// saturates to the codeword 6 (both checked on the GPU for every such fp32 c,
// both signs and slots; the first for every u).
__device__ __forceinline__ uint32_t encode8_sr_e2m1_w(const float w[8], uint32_t rnd0, uint32_t rnd1) {
    float c[8];
    #pragma unroll
    for (int j = 0; j < 8; ++j)
        c[j] = __uint_as_float((__float_as_uint(w[j]) & 0x80000000u) | __float_as_uint(__builtin_ceilf(fabsf(w[j]))));
    return encode8_sr_e2m1_short(c, rnd0, rnd1, 0x1p23f);
}

__device__ __forceinline__ uint32_t encode1_rtn_uniform(float v) {
    const float vc = fminf(fabsf(v), 7.0f);
    const uint32_t k = __float_as_uint(vc + 8388608.0f) - 0x4B000000u;   // RNE to integer
    return k | sign_nibble(v);
}

// floor(1/2 - a): v_cvt_rpi_i32_f32 (floor(x + 1/2)) of x = -a, one instruction.
// Checked against floor in double precision for every fp32 a in [0, 1792].
__device__ __forceinline__ int32_t floor_half_minus(float a) {
    int32_t r;
    asm("v_cvt_rpi_i32_f32_e64 %0, -%1" : "=v"(r) : "v"(a));
    return r;
}

// SR on the uniform grid, from w = 256 v: k = ceil(m - c) with m = min(|v|, 7)
// and c = (u + 1/2)/256.  For integer k, k >= m - c exactly when
// 256 k + u >= ceil(256 m - 1/2) = E, so k = ceil((E - u)/256) =
// (E + 255 - u) >> 8, where E = -floor(1/2 - 256 m) is one conversion of
// 256 m = min(|w|, 1792) and 255 - u is a byte of the inverted random word.
// The results t = E + 255 - u lie in [0, 2047], so k is byte 1 of t: byte
// permutes gather the even and the odd elements' k into two words that one
// shift-or merges into nibbles, and the eight sign bits are moved to bit 3 of
// their nibbles with byte permutes.  A NaN w gives an unspecified magnitude
// (callers zero the codes of blocks with a non-finite value).
__device__ __forceinline__ uint32_t encode8_sr_uniform_w(const float w[8], uint32_t rnd0, uint32_t rnd1) {
    const uint32_t n0 = ~rnd0, n1 = ~rnd1;   // bytes 255 - u
    uint32_t t[8];
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t nu = ((j < 4 ? n0 : n1) >> (8 * (j & 3))) & 0xFFu;
        const float x = __builtin_elementwise_minimum(fabsf(w[j]), 1792.0f);
        t[j] = nu - (uint32_t)floor_half_minus(x);
    }
    const uint32_t e = __builtin_amdgcn_perm(t[2], t[0], 0x0C0C0501u) | __builtin_amdgcn_perm(t[6], t[4], 0x05010C0Cu);
    const uint32_t o = __builtin_amdgcn_perm(t[3], t[1], 0x0C0C0501u) | __builtin_amdgcn_perm(t[7], t[5], 0x05010C0Cu);
    const uint32_t* b = reinterpret_cast<const uint32_t*>(w);
    // byte 3 of a float holds its sign at bit 7: odd elements' sign bytes into
    // bytes 0..3 give bits 7, 15, 23, 31; even elements', shifted down by 4, bits 3, 11, 19, 27
    const uint32_t so = __builtin_amdgcn_perm(b[3], b[1], 0x0C0C0703u) | __builtin_amdgcn_perm(b[7], b[5], 0x07030C0Cu);
    const uint32_t se = (__builtin_amdgcn_perm(b[2], b[0], 0x0C0C0703u) | __builtin_amdgcn_perm(b[6], b[4], 0x07030C0Cu)) >> 4;
    return ((o << 4) | e) | (so & 0x80808080u) | (se & 0x08080808u);
}

__device__ __forceinline__ uint32_t encode1_guided_uniform(float v, uint32_t b) {
    const float vc = fminf(fabsf(v), 7.0f);
    const float fl = __builtin_floorf(vc);
    const uint32_t klo = (uint32_t)fl;
    const uint32_t off = vc != fl ? 1u : 0u;
    const uint32_t k = klo + (((klo ^ b) & 1u) & off);
    return k | sign_nibble(v);
}

// rnd: 8 random bytes for SR (rnd0 bytes 0..3 -> elements 0..3, rnd1 -> 4..7);
// gbits: 8 guide bits for guided.  SHORT: every |v| has at most 14
// significant bits, so E2M1 SR may give v to the hardware convert as it is
// (otherwise 2^23 v goes through encode8_sr_e2m1_w).  scale: a power of two
// the E2M1 RTN and short SR paths divide v by inside the convert; every other
// path takes already scaled values (scale 1).
template <int GRID, int MODE, bool SHORT = false>
__device__ __forceinline__ uint32_t encode8(const float v[8], uint32_t rnd0, uint32_t rnd1,
                                            uint32_t gbits, float scale = 1.0f) {
    if constexpr (GRID == 0 && MODE == MODE_RTN) {
        return pack_rne8(v, scale);
    } else if constexpr (GRID == 0 && MODE == MODE_GUIDED) {
        return encode8_guided_e2m1(v, gbits);
    } else if constexpr (GRID == 0 && MODE == MODE_SR && SHORT) {
        return encode8_sr_e2m1_short(v, rnd0, rnd1, scale);
    } else if constexpr (GRID == 0 && MODE == MODE_SR) {
        float w[8];
        #pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = v[j] * 0x1p23f;   // exact, or an overflow that saturates
        return encode8_sr_e2m1_w(w, rnd0, rnd1);
    } else if constexpr (MODE == MODE_SR) {
        float w[8];
        #pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = v[j] * 256.0f;   // exact, or an overflow that saturates
        return encode8_sr_uniform_w(w, rnd0, rnd1);
    } else {
        uint32_t w = 0;
        #pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t nib;
            if constexpr (MODE == MODE_RTN) nib = encode1_rtn_uniform(v[j]);
            else nib = encode1_guided_uniform(v[j], (gbits >> j) & 1u);
            w |= nib << (4 * j);
        }
        return w;
    }
}

// ---------------------------------------------------------------- decode
// G[k] with sign for 8 packed codes: E2M1 via the hardware decode (exact),
// uniform via integers.
template <int GRID>
__device__ __forceinline__ void decode8(uint32_t w, float g[8]) {
    if constexpr (GRID == 0) {
        v2f a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        v2f b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        v2f c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
        v2f d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        g[0] = a[0]; g[1] = a[1]; g[2] = b[0]; g[3] = b[1];
        g[4] = c[0]; g[5] = c[1]; g[6] = d[0]; g[7] = d[1];
    } else {
        #pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t nib = (w >> (4 * j)) & 0xFu;
            g[j] = __uint_as_float(__float_as_uint((float)(nib & 7u)) | ((nib & 8u) << 28));
        }
    }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Dequantized values of one 16-group from its codes and block scale code:
// NVFP4 RN(RN(G*d)*s_t) (G*d exact), MXFP4 G*2^(code-127); returns false for a
// NaN scale code.
template <int FMT, int GRID>
__device__ __forceinline__ bool dequant16(uint32_t c0, uint32_t c1, uint32_t sc, float ts, float v[16]) {
    decode8<GRID>(c0, v);
    decode8<GRID>(c1, v + 8);
    if constexpr (FMT == 0) {
        const float d = e4m3_decode(sc);
        #pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = (v[j] * d) * ts;
        return (sc & 0x7Fu) != 0x7Fu;
    } else {
        const float s2 = mx_scale(sc);
        #pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = v[j] * s2;
        return sc != 0xFFu;
    }
}

// Same for one half-group (8 codes in one dword).
template <int FMT, int GRID>
__device__ __forceinline__ bool dequant8(uint32_t c, uint32_t sc, float ts, float v[8]) {
    decode8<GRID>(c, v);
    if constexpr (FMT == 0) {
        const float d = e4m3_decode(sc);
        #pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = (v[j] * d) * ts;
        return (sc & 0x7Fu) != 0x7Fu;
    } else {
        const float s2 = mx_scale(sc);
        #pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = v[j] * s2;
        return sc != 0xFFu;
    }
}

// 8 fp32 -> 8 bf16 (RNE) as 4 dwords; canonical quiet NaN when !ok.
__device__ __forceinline__ void to_bf16x8(const float v[8], bool ok, uint32_t o[4]) {
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        bf16x2 h = __builtin_convertvector((v2f){v[2 * j], v[2 * j + 1]}, bf16x2);
        o[j] = ok ? __builtin_bit_cast(uint32_t, h) : 0x7FC07FC0u;
    }
}

// 16 fp32 -> 16 bf16 (RNE) as 8 dwords; canonical quiet NaN when !ok.
__device__ __forceinline__ void to_bf16x16(const float v[16], bool ok, uint32_t o[8]) {
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        bf16x2 h = __builtin_convertvector((v2f){v[2 * j], v[2 * j + 1]}, bf16x2);
        o[j] = ok ? __builtin_bit_cast(uint32_t, h) : 0x7FC07FC0u;
    }
}

// ---------------------------------------------------------------- RHT16
// Sylvester-ordered butterfly, stages h = 1, 2, 4, 8, each sum rounded to fp32.
__device__ __forceinline__ void butterfly16(float a[16]) {
    #pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
        #pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i & h) continue;
            const float s = a[i] + a[i + h];
            const float d = a[i] - a[i + h];
            a[i] = s;
            a[i + h] = d;
        }
    }
}

// Sign mask of the RHT diagonal: bit j of word 0 of Philox(key = seed, counter
// (0,0,1,0)).  The seed is the same for every lane; written with 32-bit
// products so the compiler keeps the whole generator on the scalar unit.
__device__ __forceinline__ uint32_t rht_sign_mask(uint64_t seed) {
    uint32_t x0 = 0u, x1 = 0u, x2 = 1u, x3 = 0u;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    #pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint32_t hi0 = __umulhi(x0, 0xD2511F53u), lo0 = x0 * 0xD2511F53u;
        const uint32_t hi2 = __umulhi(x2, 0xCD9E8D57u), lo2 = x2 * 0xCD9E8D57u;
        const uint32_t y0 = hi2 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
        x1 = lo2;
        x3 = lo0;
        x0 = y0;
        x2 = y2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return x0 & 0xFFFFu;
}

// 16 bf16 (8 dwords) -> fp32, with optional forward RHT (signs first).
// QUARTER = false leaves out the final exact multiply by 1/4: callers fold it
// into their block scale.  (The butterfly sums of bf16 inputs are multiples of
// 2^-133, so a * 1/4 is always exact; it never needs to be rounded.)
template <bool RHT, bool QUARTER = true>
__device__ __forceinline__ void widen16(const uint32_t w[8], uint32_t signs, float y[16]) {
    if constexpr (RHT) {
        // the diagonal's sign bits are the same for every lane: widening and sign
        // flip in one instruction per element (adding 2^31 flips bit 31)
        #pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t slo = ((signs >> (2 * j)) & 1u) << 31, shi = ((signs >> (2 * j + 1)) & 1u) << 31;
            uint32_t lo;
            asm("v_lshl_add_u32 %0, %1, 16, %2" : "=v"(lo) : "v"(w[j]), "s"(slo));
            y[2 * j] = __uint_as_float(lo);
            y[2 * j + 1] = __uint_as_float((w[j] & 0xFFFF0000u) ^ shi);
        }
        butterfly16(y);
        if constexpr (QUARTER) {
            #pragma unroll
            for (int j = 0; j < 16; ++j) y[j] = y[j] * 0.25f;
        }
    } else {
        #pragma unroll
        for (int j = 0; j < 8; ++j) {
            y[2 * j] = bf16_lo(w[j]);
            y[2 * j + 1] = bf16_hi(w[j]);
        }
    }
}

// ---------------------------------------------------------------- lane exchange
// quad_perm DPP moves within each row of four lanes: [1,0,3,2] swaps pair
// partners, [2,3,0,1] swaps the two pairs.  Callers make every lane execute
// them (a lane reading an inactive partner gets 0).
__device__ __forceinline__ uint32_t dpp_swap1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_swap2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
}

// Pair exchange: lane q of a pair holds a (slot 2k) and b (slot 2k+1) and
// returns lo = its a (q = 0) or the partner's b (q = 1), hi = the partner's a
// (q = 0) or its b (q = 1).  Each lane sends the one it gives away (b for
// q = 0, a for q = 1).  The received value feeds both selects, so the DPP move
// is computed by every lane: a DPP move placed under a lane-dependent branch
// would read inactive partner lanes.
__device__ __forceinline__ void pair_exchange(const uint32_t a[4], const uint32_t b[4], uint32_t q,
                                              uint32_t lo[4], uint32_t hi[4]) {
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t r = dpp_swap1(q ? a[j] : b[j]);
        lo[j] = q ? r : a[j];
        hi[j] = q ? b[j] : r;
    }
}

// Largest |bf16| bit pattern of 16 values (8 dwords) with sign bits cleared;
// >= 0x7F80 means the group holds a non-finite value.  Packed 16-bit max.

__device__ __forceinline__ uint32_t amax_bits16(const uint32_t w[8]) {
    u16x2 m = __builtin_bit_cast(u16x2, w[0] & 0x7FFF7FFFu);
    #pragma unroll
    for (int j = 1; j < 8; ++j)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// ---------------------------------------------------------------- grouped launches
// The part t of a grouped launch that workgroup b belongs to: start[t] <= b <
// start[t + 1], for n parts (n <= N) with non-decreasing starts.  Counting the
// starts at or below b over all N entries at once lets them come in with wide
// scalar loads; a scan that stops at the first start past b made one dependent
// load per part before the workgroup could load anything else.
template <int N>
__device__ __forceinline__ uint32_t group_of(const uint32_t (&start)[N + 1], uint32_t n, uint32_t b) {
    uint32_t t = 0;
    #pragma unroll
    for (int i = 1; i < N; ++i) t += ((uint32_t)i < n && b >= start[i]) ? 1u : 0u;
    return t;
}

// ---------------------------------------------------------------- cross-workgroup maximum
// Maximum of m over a workgroup of WAVES waves, valid in thread 0.  red: WAVES
// words of LDS.
template <int WAVES = 4>
__device__ __forceinline__ uint32_t wg_max_t0(uint32_t m, uint32_t* red) {
    #pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        #pragma unroll
        for (int i = 1; i < WAVES; ++i) m = max(m, red[i]);
    }
    return m;
}

// NVFP4 tensor scale from the bits of the largest finite |y|: amax / RN(Gmax * 448),
// or 1 for an all-zero tensor.
__device__ __forceinline__ float ts_from_amax(uint32_t amax_bits, float gmax448) {
    const float a = __uint_as_float(amax_bits);
    return a == 0.0f ? 1.0f : a / gmax448;
}

// Cross-workgroup reduction without atomics.  Workgroup b of a launch stores
// tag << 32 | m in word b of a workspace; one workgroup reads every word until
// all carry the call's tag.  The stores and loads are relaxed and agent-scope:
// performed at the device's point of coherence, not held in one XCD's L2.  The
// tag is the workspace's epoch + 1, and only the gathering workgroup advances
// the epoch, after it has seen every word tagged, when every workgroup has read
// the epoch already; so a word from an earlier call never passes for one of
// this call (until the 32-bit epoch wraps), and all-zero words are a valid start.
__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t v) { return (uint64_t)tag << 32 | v; }

// The workspace's 64-bit state word: the epoch in its low half and, in its high
// half, the mark of the last launch whose wait gave up (0 after a launch that
// did not).  A launch's mark comes from the address of its dispatch packet,
// which differs between queues and between launches on a queue until its ring
// of packets wraps, graph replays included (never 0).
__device__ __forceinline__ uint32_t launch_mark() {
    const uintptr_t a = reinterpret_cast<uintptr_t>(__builtin_amdgcn_dispatch_ptr());
    return ((uint32_t)(a >> 6) & 0x7FFFFFFFu) + 1u;   // packets are 64 bytes
}

// A call as its workgroup sees it at the start: its tag (the epoch + 1) and
// whether its own launch has already given up.  When a wait gives up, the
// gathering workgroup advances the epoch without knowing that every workgroup
// of the launch has read it; one that starts later would read the new epoch
// and tag its word with the next call's tag, which that call's gather could
// take for its own.  The mark in the same word tells such a workgroup that its
// launch is over: it stores nothing.  (A later launch whose packet lands in the
// marked slot before any call has succeeded on this workspace since is taken
// for that launch: it gives s_t = NaN, never a wrong one, and the call after it
// proceeds.)
struct CallState {
    uint32_t epoch, tag;
    bool late;
};
__device__ __forceinline__ CallState call_state(const uint32_t* state) {
    const uint64_t w = load_agent(reinterpret_cast<const uint64_t*>(state));
    return CallState{(uint32_t)w, (uint32_t)w + 1u, (uint32_t)(w >> 32) == launch_mark()};
}
// The gathering workgroup's last store: the next epoch, and this launch's mark
// if its wait gave up.
__device__ __forceinline__ void end_call(uint32_t* state, uint32_t epoch, bool gave_up) {
    store_agent(reinterpret_cast<uint64_t*>(state), (uint64_t)(gave_up ? launch_mark() : 0u) << 32 | (epoch + 1u));
}

// Polls before a wait gives up, by default: 2^20 loads, about a second.  The
// launches take the limit as an argument (fp4_set_wait_limit).
constexpr uint32_t kGatherPolls = 1u << 20;

// This thread's share of the gather: the largest low half of words i = threadIdx.x
// + THREADS k < n (at most MAXN words), once all of them carry `tag`; each round
// loads them all at once.  Returns 0xFFFFFFFF if they are not all tagged within
// `polls` rounds (the maxima are finite float bits, never that value).
template <uint32_t MAXN, uint32_t THREADS>
__device__ __forceinline__ uint32_t gather_max(const uint64_t* words, uint32_t n, uint32_t tag, uint32_t polls) {
    constexpr uint32_t kPer = (MAXN + THREADS - 1) / THREADS;
    for (uint32_t r = 0; r < polls; ++r) {
        uint64_t v[kPer];
        #pragma unroll
        for (uint32_t k = 0; k < kPer; ++k) {
            const uint32_t i = threadIdx.x + THREADS * k;
            v[k] = i < n ? load_agent(words + i) : tagged(tag, 0u);
        }
        bool all = true;
        uint32_t g = 0;
        #pragma unroll
        for (uint32_t k = 0; k < kPer; ++k) {
            all = all && (uint32_t)(v[k] >> 32) == tag;
            g = max(g, (uint32_t)v[k]);
        }
        if (all) return g;
        __builtin_amdgcn_s_sleep(1);
    }
    return 0xFFFFFFFFu;
}

}  // namespace fp4q
