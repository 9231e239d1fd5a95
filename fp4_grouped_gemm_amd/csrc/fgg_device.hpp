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

// e4m3 code of an fp32 value (host and device).
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

// fl32(x / s) as far as the e4m3 code of it is concerned, given r = rcp(s).
// The hardware reciprocal is within one ulp, so q = x·r lies within about 3.5 ulps of
// the correctly rounded quotient.  That neighbourhood can change the e4m3 code only
// when q sits near a rounding midpoint (the 20 bits below the 3 kept mantissa bits
// near 0x80000: lanes within 8 ulps of it), below the normal e4m3 range (a finer grid),
// or far above 448 / not finite (degenerate scales); those lanes take the IEEE
// division, every other lane's code equals that of the exact quotient (checked on
// 2^30 uniform and 2^30 midpoint-adjacent (x, s) pairs on MI355X: no difference).
// q = x·r keeps x's sign, also for zero.  Requires s > 0.
__device__ inline float e4m3_quotient(float x, float s, float r) {
  float q = x * r;
  const uint32_t a = __float_as_uint(q) & 0x7FFFFFFFu;
  const bool risky = (a < 0x3C800000u) | ((a & 0xFFFFFu) - 0x7FFF8u < 16u) | (a > 0x43E80000u);
  if (__builtin_expect(risky, 0)) q = x / s;
  return q;
}

// Four e4m3 codes packed little-endian (v0 in the low byte), by the gfx950
// conversion instruction (OCP e4m3, round to nearest even) after clamping to
// the finite range; equal to e4m3_encode on every finite input.
__device__ inline uint32_t e4m3_pack4(float v0, float v1, float v2, float v3) {
  v0 = __builtin_amdgcn_fmed3f(v0, -448.0f, 448.0f);
  v1 = __builtin_amdgcn_fmed3f(v1, -448.0f, 448.0f);
  v2 = __builtin_amdgcn_fmed3f(v2, -448.0f, 448.0f);
  v3 = __builtin_amdgcn_fmed3f(v3, -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
  return (uint32_t)w;
}

// e^-g from the hardware base-2 exponential: -g·log2(e) is formed as hi + lo
// (log2(e) split into fp32 hi and lo parts, the product's rounding error
// recovered with an FMA) and 2^(hi + lo) = 2^hi · (1 + lo·ln 2) to first order,
// which keeps the result within a few ulps; overflow gives +inf, underflow 0.
__device__ inline float exp_neg(float g) {
  constexpr float kLog2eHi = 1.44269502162933349609375f;   // fp32 nearest to log2(e)
  constexpr float kLog2eLo = 1.92596298909109e-08f;        // log2(e) - kLog2eHi
  constexpr float kLn2 = 0.693147180559945309f;
  const float x = -g * kLog2eHi;
  const float x_lo = __builtin_fmaf(-g, kLog2eHi, -x) - g * kLog2eLo;
  const float e = __builtin_amdgcn_exp2f(x);
  return __builtin_fmaf(e, x_lo * kLn2, e);
}

// a / d for d >= 1 (SiLU denominators): reciprocal and one Newton step,
// within about one ulp; d is clamped finite so that a huge denominator gives 0.
__device__ inline float div_by_ge1(float a, float d) {
  d = __builtin_fminf(d, 3.0e38f);
  const float r = __builtin_amdgcn_rcpf(d);
  float t = a * r;
  const float e = __builtin_fmaf(-t, d, a);
  return __builtin_fmaf(e, r, t);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__host__ __device__ inline uint16_t bf16_bits_rne(float v) {
  uint32_t b;
  __builtin_memcpy(&b, &v, 4);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Two fp32 values -> packed bf16 bits (a in the low half), round to nearest even, by the
// gfx950 conversion instruction (v_cvt_pk_bf16_f32).  Measured on MI355X against
// bf16_bits_rne on all 2^32 fp32 bit patterns: equal for every non-NaN input, NaN stays
// NaN.
__device__ inline uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
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

// Eight consecutive elements (bf16 or fp32) as fp32, from 16- or 32-byte loads.
template <bool BF16>
__device__ inline void load8(const void* base, int64_t idx, float* f) {
  if (BF16) {
    const uint4 u = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
      f[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    const float4 a = p[0], b = p[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// ---------------------------------------------------------------------------
// gfx950's direct global->LDS loads and the waits the GEMM pipelines count by hand.
// The LDS destination is M0 (+ 16 or 4 bytes per lane, consecutive lanes consecutive);
// M0 is saved and restored around the load.  The source is a wave-uniform base (an
// SGPR pair) plus a per-lane 32-bit offset.  Their completion is counted in vmcnt like
// any vector-memory load.

// 16 bytes per lane from sbase + voff into LDS at m0 + 16 * lane.
__device__ inline void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// 4 bytes per lane from sbase + voff into LDS at m0 + 4 * lane.
__device__ inline void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// s_waitcnt immediate (gfx9 encoding) for lgkmcnt(0) with vmcnt and expcnt left at their maxima
constexpr int kLgkmZero = 0xC07F;

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ inline void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// A pointer the compiler is told is the same in every lane (it is: built from
// workgroup-uniform values), so that it can be a DMA instruction's scalar base.
template <class T>
__device__ inline T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace fgg
