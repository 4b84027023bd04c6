// The Q8_0 / Q4_0 rounding chain of include/kvattn.h ("Quantisation"), shared
// by the page quantiser and the decode kernel's fused append so both write the
// same bytes. Every step is one IEEE binary32 operation (round to nearest
// even) or a binary32 -> binary16 conversion; none of them may be contracted.
#pragma once

#include "common.hpp"

namespace kvattn {

// Q8_0 block scale from the block's largest magnitude: RN16(RN32(amax / 127)).
__device__ __forceinline__ _Float16 q8_scale(float amax) {
#pragma clang fp contract(off)
  return (_Float16)(amax / 127.0f);
}

// Q8_0 code byte of x under inv = RN32(1 / d): clamp(rint(RN32(x * inv)), -127, 127).
__device__ __forceinline__ uint32_t q8_code(float x, float inv) {
#pragma clang fp contract(off)
  const float r = fminf(fmaxf(rintf(x * inv), -127.0f), 127.0f);
  return (uint32_t)(int)r & 0xFFu;
}

// Q4_0 block scale from the signed element of largest magnitude m: RN16(RN32(-m / 8)).
__device__ __forceinline__ _Float16 q4_scale(float m) {
#pragma clang fp contract(off)
  return (_Float16)((-m) / 8.0f);
}

// Q4_0 code (0..15) of y under inv = RN32(1 / d): clamp(rint(RN32(y * inv)), -8, 7) + 8.
__device__ __forceinline__ uint32_t q4_code(float y, float inv) {
#pragma clang fp contract(off)
  const float r = fminf(fmaxf(rintf(y * inv), -8.0f), 7.0f);
  return (uint32_t)((int)r + 8);
}

// Q5_1 block scale from the block's extremes: RN16(RN32((mx - mn) / 31)).
__device__ __forceinline__ _Float16 q5_scale(float mx, float mn) {
#pragma clang fp contract(off)
  return (_Float16)((mx - mn) / 31.0f);
}

// Q5_1 code (0..31) of x under the stored minimum m and inv = RN32(1 / d):
// clamp(rint(RN32(RN32(x - m) * inv)), 0, 31).
__device__ __forceinline__ uint32_t q5_code(float x, float m, float inv) {
#pragma clang fp contract(off)
  const float r = fminf(fmaxf(rintf((x - m) * inv), 0.0f), 31.0f);
  return (uint32_t)(int)r;
}

// Bit of dim 8w + k (k = 0..7) in the byte of fifth bits of word w.
__device__ __forceinline__ int k5_hi_bit(int k) { return (k >> 1) + 4 * (k & 1); }

// Bit offset of slot j (0..7) inside a V word: slot pairs share a byte.
__device__ __forceinline__ int v_slot_bit(int j) { return 4 * (j >> 1) + 16 * (j & 1); }

}  // namespace kvattn
