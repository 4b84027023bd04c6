// Shared device definitions for libkvattn (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvattn {

constexpr int D = 256;            // head_dim
constexpr int PAGE = 128;         // tokens per page
constexpr int K_REC = 34816;      // bytes per (page, KV head) key record
constexpr int V_REC = 18432;      // bytes per (page, KV head) value record, Q4_0 values
constexpr int V8_REC = 34816;     // the same with Q8_0 values (laid out like a key record)
constexpr int K4_REC = 18432;     // bytes per key record with Q4_0 keys
constexpr int K4_SCALE_OFF = 16384;
constexpr int K5_REC = 24576;     // bytes per key record with Q5_1 keys
constexpr int K5_HI_OFF = 16384;  // fifth bits: byte t*32 + w for dims 8w..8w+7
constexpr int K5_D_OFF = 20480;   // scales d
constexpr int K5_M_OFF = 22528;   // minimums m
constexpr int K_SCALE_OFF = 32768;
constexpr int V_SCALE_OFF = 16384;
// Key record size and scale offset by key type (0 Q8_0, 1 Q4_0, 2 Q5_1).
template <int KT> constexpr int KREC_OF = KT == 0 ? K_REC : KT == 1 ? K4_REC : K5_REC;
template <int KT> constexpr int KSCALE_OF = KT == 0 ? K_SCALE_OFF : KT == 1 ? K4_SCALE_OFF : K5_D_OFF;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ uint16_t f16_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_value(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// 16x16x32 f16 matrix-core product, fp32 accumulate.
__device__ __forceinline__ floatx4 mfma16(half8_t a, half8_t b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }
__device__ __forceinline__ uint32_t as_u32(half2_t x) { return __builtin_bit_cast(uint32_t, x); }

// Eight signed int8 codes (two dwords) -> eight f16 values code*d, where the
// f16 pair d2 holds the block scale twice. Bytes are offset to unsigned
// (xor 0x80), placed under the exponent byte 0x64 (f16 1024 + byte), and the
// 1152 offset is removed exactly before the scale multiply.
__device__ __forceinline__ half8_t k_codes_to_f16(uint32_t w0, uint32_t w1, half2_t d2) {
  const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t y0 = w0 ^ 0x80808080u, y1 = w1 ^ 0x80808080u;
  half2_t a = (as_h2(__builtin_amdgcn_perm(0x64646464u, y0, 0x04010400u)) - off) * d2;
  half2_t b = (as_h2(__builtin_amdgcn_perm(0x64646464u, y0, 0x04030402u)) - off) * d2;
  half2_t c = (as_h2(__builtin_amdgcn_perm(0x64646464u, y1, 0x04010400u)) - off) * d2;
  half2_t e = (as_h2(__builtin_amdgcn_perm(0x64646464u, y1, 0x04030402u)) - off) * d2;
  half8_t r = {a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
  return r;
}

// Eight int8 codes (two words, byte order) -> eight exact f16 values
// (Q8_0 values: the scale is applied elsewhere).
__device__ __forceinline__ half8_t v8_codes_to_f16(uint32_t w0, uint32_t w1) {
  const half2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t y0 = w0 ^ 0x80808080u, y1 = w1 ^ 0x80808080u;
  const half2_t a = as_h2(__builtin_amdgcn_perm(0x64646464u, y0, 0x04010400u)) - off;
  const half2_t b = as_h2(__builtin_amdgcn_perm(0x64646464u, y0, 0x04030402u)) - off;
  const half2_t c = as_h2(__builtin_amdgcn_perm(0x64646464u, y1, 0x04010400u)) - off;
  const half2_t e = as_h2(__builtin_amdgcn_perm(0x64646464u, y1, 0x04030402u)) - off;
  half8_t r = {a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
  return r;
}

// Nibble unpacking. A word holds eight 4-bit codes; pair p (the f16 pair
// 2p, 2p+1) is the nibbles at bits 4p and 16 + 4p. A pair at bits 0-3/16-19
// is put under the exponent of 2^10, where the mantissa step is 1: the f16 is
// 1024 + code. A pair at bits 4-7/20-23 is put, without a shift, under the
// exponent of 2^6, where the step is 1/16, so the code four bits up reads as
// 64 + code. One shift by 8 brings the other two pairs to those places, so a
// word takes five bitwise ops (the masks in VGPRs, the exponents in SGPRs).
constexpr uint32_t NIB_LO = 0x000F000Fu, NIB_HI = 0x00F000F0u;
constexpr uint32_t EXP_1024 = 0x64006400u, EXP_64 = 0x54005400u;

// One V word -> eight exact f16 values (code - 8) in pair order.
__device__ __forceinline__ half8_t v_codes_to_f16_m(uint32_t w, uint32_t mlo, uint32_t mhi) {
  const half2_t off_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t off_hi = {(_Float16)72.0f, (_Float16)72.0f};
  const uint32_t t = w >> 8;
  const half2_t p0 = as_h2((w & mlo) | EXP_1024) - off_lo;
  const half2_t p1 = as_h2((w & mhi) | EXP_64) - off_hi;
  const half2_t p2 = as_h2((t & mlo) | EXP_1024) - off_lo;
  const half2_t p3 = as_h2((t & mhi) | EXP_64) - off_hi;
  half8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}
__device__ __forceinline__ half8_t v_codes_to_f16(uint32_t w) {
  return v_codes_to_f16_m(w, NIB_LO, NIB_HI);
}

// One Q4_0 key word (dims 8w..8w+7, nibble order of the V words) -> eight
// f16 values d * (code - 8); d2 holds the block scale in both halves.
__device__ __forceinline__ half8_t k4_codes_to_f16(uint32_t w, uint32_t mlo, uint32_t mhi, half2_t d2) {
  const half8_t d8 = __builtin_shufflevector(d2, d2, 0, 1, 0, 1, 0, 1, 0, 1);
  return v_codes_to_f16_m(w, mlo, mhi) * d8;
}

// One Q5_1 key word (low nibbles as a Q4_0 key word) and its byte e of fifth
// bits (dim 8w + 2p at bit p, 8w + 2p + 1 at bit 4 + p) -> eight f16 values
// d * code + m (one rounding); d2, m2 hold the block's d and m in both halves.
// The fifth bit goes just above its nibble: bit 4 (16 + 4) under 2^10, bit 8
// (24) under 2^6, where the 5-bit code still reads 1024 + code or 64 + code.
// e * 0x10010 puts e's bits 0-3 at bits 4-7 and bits 4-7 at bits 20-23.
__device__ __forceinline__ half8_t k5_codes_to_f16(uint32_t w, uint32_t e, uint32_t mlo, uint32_t mhi,
                                                   half2_t d2, half2_t m2) {
  const uint32_t hs = e * 0x10010u;
  const uint32_t t = w >> 8;
  const half2_t off_lo = {(_Float16)1024.0f, (_Float16)1024.0f};
  const half2_t off_hi = {(_Float16)64.0f, (_Float16)64.0f};
  const uint32_t c0 = ((w & mlo) | EXP_1024) | (hs & 0x00100010u);
  const uint32_t c1 = ((w & mhi) | EXP_64) | ((hs << 3) & 0x01000100u);
  const uint32_t c2 = ((t & mlo) | EXP_1024) | ((hs >> 2) & 0x00100010u);
  const uint32_t c3 = ((t & mhi) | EXP_64) | ((hs << 1) & 0x01000100u);
  const half2_t v0 = __builtin_elementwise_fma(as_h2(c0) - off_lo, d2, m2);
  const half2_t v1 = __builtin_elementwise_fma(as_h2(c1) - off_hi, d2, m2);
  const half2_t v2 = __builtin_elementwise_fma(as_h2(c2) - off_lo, d2, m2);
  const half2_t v3 = __builtin_elementwise_fma(as_h2(c3) - off_hi, d2, m2);
  half8_t r = {v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
  return r;
}
__device__ __forceinline__ half8_t k5_codes_to_f16(uint32_t w, uint32_t e, half2_t d2, half2_t m2) {
  return k5_codes_to_f16(w, e, NIB_LO, NIB_HI, d2, m2);
}

__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load16_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint32_t load4_nt(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// Reductions over the lanes l, l^16, l^32, l^48 (the four 16-lane rows of a
// wave), with the gfx950 row-swap permutes. v_permlane16_swap of a value
// with itself yields rows (0,0,2,2) in one operand and (1,1,3,3) in the
// other; v_permlane32_swap yields (0,1,0,1) and (2,3,2,3). Combining the two
// halves each time reduces across rows. (The result elements are copied to
// scalars before any bit cast: a bit cast applied to an element of the
// returned pair reads element 0 whatever the index.)
__device__ __forceinline__ float row_swap_combine16(float x, bool is_max) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float p = __builtin_bit_cast(float, a0), q = __builtin_bit_cast(float, a1);
  return is_max ? fmaxf(p, q) : p + q;
}
__device__ __forceinline__ float row_swap_combine32(float x, bool is_max) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float p = __builtin_bit_cast(float, a0), q = __builtin_bit_cast(float, a1);
  return is_max ? fmaxf(p, q) : p + q;
}
// x combined over its group of eight lanes (8k .. 8k+7) by DPP moves: swap
// neighbours, swap pairs, then mirror the half row. Each step adds (or takes
// the max of) the same two values on both lanes of a pair, so all eight lanes
// end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// The value held by a partner lane in the same group of eight: lane l ^ 1
// (o = 1), l ^ 2 (o = 2), or 7 - l within the group (o = 4, row_half_mirror,
// which pairs every lane with one of the other quad). Three steps with o = 1,
// 2, 4 reduce any commutative, associative selection over the eight lanes
// onto all of them, as three xor shuffles would. o must be a constant.
__device__ __forceinline__ uint32_t peer8(uint32_t x, int o) {
  return o == 1   ? (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false)
         : o == 2 ? (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false)
                  : (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false);
}
__device__ __forceinline__ float peer8(float x, int o) {
  return __builtin_bit_cast(float, peer8(__builtin_bit_cast(uint32_t, x), o));
}
__device__ __forceinline__ int peer8(int x, int o) { return (int)peer8((uint32_t)x, o); }

__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  return fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
}
__device__ __forceinline__ float group8_sum(float x) {
  x = x + dpp_f<0xB1>(x);
  x = x + dpp_f<0x4E>(x);
  return x + dpp_f<0x141>(x);
}
__device__ __forceinline__ float wave_max_xor_16_32(float x) {
  return row_swap_combine32(row_swap_combine16(x, true), true);
}
__device__ __forceinline__ float wave_sum_xor_16_32(float x) {
  return row_swap_combine32(row_swap_combine16(x, false), false);
}

}  // namespace kvattn
