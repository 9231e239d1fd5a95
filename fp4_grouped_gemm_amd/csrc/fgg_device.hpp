// Device helpers shared by the fgg kernels (gfx950 only).
//
// Encoders are written from the format definitions:
//   e4m3 (OCP FP8 "FN"): bias 7, 3 mantissa bits, largest finite 448, no inf
//     ([DeepGEMM] bhfrc.com/news/60438 §2.1, format table);
//   E2M1: bias 1, 1 mantissa bit, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}
//     ([Infra] "腾讯 AI Infra", Q "FP4量化是什么", FP4 format table).
// Rounding is to nearest with ties to the even code; finite values beyond the
// largest magnitude saturate; the sign is always kept (also for zero).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// e4m3 code of an fp32 value.  Host and device (the host build is used by a
// CPU unit test of the encoder).
__host__ __device__ inline uint8_t e4m3_encode(float v) {
  uint32_t bits;
  __builtin_memcpy(&bits, &v, 4);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7FFFFFFFu;
  if (abits > 0x7F800000u) return 0x7F;               // NaN
  if (abits >= 0x43E00000u) return (uint8_t)(sign | 0x7E);   // |v| >= 448: saturate
  if (abits < 0x3C800000u) {                          // |v| < 2^-6: subnormal grid of 2^-9
    float a;
    __builtin_memcpy(&a, &abits, 4);
    float m = a * 512.0f;                             // exact (power-of-two scaling)
    // round half to even on [0, 8]; 8 becomes the smallest normal code 0x08
    uint32_t mi = (uint32_t)m;
    float frac = m - (float)mi;
    if (frac > 0.5f || (frac == 0.5f && (mi & 1u))) mi += 1;
    return (uint8_t)(sign | mi);
  }
  // normal: exponent E in [-6, 8]; keep 3 mantissa bits, RNE on the dropped 20 bits
  const int E = (int)(abits >> 23) - 127;
  uint32_t code = ((uint32_t)(E + 7) << 3) | ((abits >> 20) & 7u);
  const uint32_t rem = abits & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1;   // carry may bump the exponent
  if (code > 0x7E) code = 0x7E;
  return (uint8_t)(sign | code);
}

// E2M1 code (low nibble) of an fp32 value: count how many rounding
// boundaries lie below |v|; at a tie the boundary counts only when the upper
// neighbour has the even code.
__host__ __device__ inline uint32_t e2m1_encode(float v) {
  uint32_t bits;
  __builtin_memcpy(&bits, &v, 4);
  const uint32_t sign = (bits >> 28) & 0x8u;
  float a = __builtin_fabsf(v);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return sign | c;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__host__ __device__ inline uint16_t bf16_bits_rne(float v) {
  uint32_t b;
  __builtin_memcpy(&b, &v, 4);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__host__ __device__ inline float bf16_to_f32(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  __builtin_memcpy(&f, &b, 4);
  return f;
}

__host__ __device__ inline float e2m1_value(uint32_t nib) {
  // 0, .5, 1, 1.5, 2, 3, 4, 6 by the bit layout: e = (n>>1)&3, m = n&1
  const uint32_t e = (nib >> 1) & 3u, m = nib & 1u;
  float mag = (e == 0) ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (e - 1));
  return (nib & 8u) ? -mag : mag;
}

template <int W>
__device__ inline float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
  return v;
}

}  // namespace fgg
