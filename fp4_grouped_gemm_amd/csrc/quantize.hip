// Block quantization kernels: fp32/bf16 -> e4m3 or E2M1 plus block scales.
//
// Rule ([Infra] "腾讯 AI Infra", Q "量化矩阵乘的维度和流程", per-group
// quantization; [DeepGEMM] bhfrc.com/news/60438 §5.2, scale = max|x| / 448):
// one scale per block from the block's largest magnitude, codes = round(x / s).
// All kernels are HBM-bound streaming passes: each thread owns a contiguous
// run of elements, loads it with 16-byte accesses, reduces the block maximum
// with lane shuffles (or LDS for 128x128 blocks) and writes packed codes.
#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

// ---------------------------------------------------------------------------
// 1 x 128 activation groups -> e4m3, scales [cols/128][rows].
// 16 threads per group (8 elements each); a 256-thread block covers 16 groups
// per step and strides over the groups of rows < min(rows, *rows_dev).
// SILU: the row holds [gate | up] (2*cols values); a = g / (1 + e^-g) * u.
template <bool BF16, bool SILU>
__global__ void __launch_bounds__(256) quant_e4m3_1x128_kernel(const void* __restrict__ x, int64_t rows,
                                                                int64_t cols, int64_t ldx,
                                                                const int32_t* __restrict__ rows_dev,
                                                                uint8_t* __restrict__ q,
                                                                float* __restrict__ scales) {
  const int64_t nkb = cols / 128;
  int64_t live_rows = rows;
  if (rows_dev) {
    const int64_t r = *rows_dev;
    live_rows = r < rows ? (r < 0 ? 0 : r) : rows;
  }
  const int64_t ngroups = live_rows * nkb;
  const int sub = threadIdx.x & 15;
  for (int64_t g0 = (int64_t)blockIdx.x * 16; g0 < ngroups; g0 += (int64_t)gridDim.x * 16) {
    const int64_t group = g0 + (threadIdx.x >> 4);
    const bool live = group < ngroups;
    const int64_t row = live ? group / nkb : 0;
    const int64_t kb = live ? group % nkb : 0;
    const int64_t col = kb * 128 + sub * 8;
    float v[8];
    if (live) {
      load8<BF16>(x, row * ldx + col, v);
      if (SILU) {
        float u[8];
        load8<BF16>(x, row * ldx + cols + col, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = div_by_ge1(v[i], 1.0f + exp_neg(v[i])) * u[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group_max<16>(amax);
    const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    const float r = __builtin_amdgcn_rcpf(s);
    if (live) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = e4m3_quotient(v[i], s, r);
      const uint32_t lo = e4m3_pack4(y[0], y[1], y[2], y[3]);
      const uint32_t hi = e4m3_pack4(y[4], y[5], y[6], y[7]);
      *reinterpret_cast<uint2*>(q + row * cols + col) = make_uint2(lo, hi);
      if (sub == 0) scales[kb * rows + row] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// 128 x 128 weight blocks -> e4m3, scales [rows/128][cols/128].
// One 256-thread block per 128x128 block; thread t owns row t/2, 64 columns.
template <bool BF16>
__global__ void __launch_bounds__(256) quant_e4m3_128x128_kernel(const void* __restrict__ x, int64_t rows,
                                                                  int64_t cols, int64_t ldx,
                                                                  uint8_t* __restrict__ q,
                                                                  float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t nkb = cols / 128;
  const int64_t rb = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int64_t row = rb * 128 + (threadIdx.x >> 1);
  const int64_t col = kb * 128 + (threadIdx.x & 1) * 64;
  float v[64];
#pragma unroll
  for (int c = 0; c < 8; ++c) load8<BF16>(x, row * ldx + col + 8 * c, v + 8 * c);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<64>(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  const float r = __builtin_amdgcn_rcpf(s);
  uint8_t* dst = q + row * cols + col;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* p = v + 16 * c + 4 * j;
      w[j] = e4m3_pack4(e4m3_quotient(p[0], s, r), e4m3_quotient(p[1], s, r), e4m3_quotient(p[2], s, r),
                        e4m3_quotient(p[3], s, r));
    }
    *reinterpret_cast<uint4*>(dst + 16 * c) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (threadIdx.x == 0) scales[rb * nkb + kb] = s;
}

// ---------------------------------------------------------------------------
// 1 x 16 groups -> packed E2M1 (8 bytes per group), fp32 scale = amax / 6,
// scales [rows][cols/16].  One thread per group.
template <bool BF16>
__global__ void __launch_bounds__(256) quant_e2m1_1x16_kernel(const void* __restrict__ x, int64_t rows,
                                                               int64_t cols, int64_t ldx,
                                                               uint8_t* __restrict__ q,
                                                               float* __restrict__ scales) {
  const int64_t ng = cols / 16;
  const int64_t group = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (group >= rows * ng) return;
  const int64_t row = group / ng, g = group % ng;
  float v[16];
  load8<BF16>(x, row * ldx + g * 16, v);
  load8<BF16>(x, row * ldx + g * 16 + 8, v + 8);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float s = (amax == 0.0f) ? 1.0f : amax / 6.0f;
  uint32_t w[2] = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_encode(v[i] / s) << (4 * (i & 7));
  *reinterpret_cast<uint2*>(q + row * (cols / 2) + g * 8) = make_uint2(w[0], w[1]);
  scales[row * ng + g] = s;
}

// ---------------------------------------------------------------------------
// 1 x 32 groups -> packed E2M1 (16 bytes per group) with an E8M0 scale byte,
// scales [rows][cols/32].  e = smallest integer with 6 * 2^e >= amax, read off
// amax's fp32 bits: amax = 1.m * 2^E gives e = E - 2 when 1.m <= 1.5, else E - 1.
__device__ inline int e8m0_exponent_of(float amax) {
  uint32_t b = __float_as_uint(amax);
  if (amax == 0.0f) return 0;
  int E;
  uint32_t mant;
  if ((b >> 23) == 0) {                        // subnormal amax: normalize
    const int lz = __clz(b) - 8;               // leading zeros within the 23-bit field + 1
    E = -126 - lz;
    mant = (b << lz) & 0x7FFFFFu;
  } else {
    E = (int)(b >> 23) - 127;
    mant = b & 0x7FFFFFu;
  }
  int e = (mant <= 0x400000u) ? E - 2 : E - 1;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

template <bool BF16>
__global__ void __launch_bounds__(256) quant_e2m1_e8m0_1x32_kernel(const void* __restrict__ x, int64_t rows,
                                                                    int64_t cols, int64_t ldx,
                                                                    uint8_t* __restrict__ q,
                                                                    uint8_t* __restrict__ scales) {
  const int64_t ng = cols / 32;
  const int64_t group = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (group >= rows * ng) return;
  const int64_t row = group / ng, g = group % ng;
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) load8<BF16>(x, row * ldx + g * 32 + 8 * c, v + 8 * c);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = e8m0_exponent_of(amax);
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i >> 3] |= e2m1_encode(ldexpf(v[i], -e)) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(q + row * (cols / 2) + g * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[row * ng + g] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------------------
const KernelInfo kInfoQuantE4m3_1x128 = {"quant_e4m3_1x128_kernel", "fgg_quantize_blockwise {E4M3,F32,1,128}",
                                         1, 128, 128, 256, 0, 0, 0, 0,
                                         (const void*)quant_e4m3_1x128_kernel<true, false>};
const KernelInfo kInfoQuantE4m3_128x128 = {"quant_e4m3_128x128_kernel", "fgg_quantize_blockwise {E4M3,F32,128,128}",
                                           128, 128, 128, 256, 0, 0, 16, 16,
                                           (const void*)quant_e4m3_128x128_kernel<true>};
const KernelInfo kInfoQuantE2m1_1x16 = {"quant_e2m1_1x16_kernel", "fgg_quantize_blockwise {E2M1X2,F32,1,16}",
                                        1, 16, 16, 256, 0, 0, 0, 0, (const void*)quant_e2m1_1x16_kernel<true>};
const KernelInfo kInfoQuantE2m1E8m0_1x32 = {"quant_e2m1_e8m0_1x32_kernel",
                                            "fgg_quantize_blockwise {E2M1X2,E8M0,1,32}", 1, 32, 32, 256, 0, 0, 0, 0,
                                            (const void*)quant_e2m1_e8m0_1x32_kernel<true>};

hipError_t launch_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ldx,
                           QuantKind kind, bool silu, const int32_t* rows_dev, void* q, void* scales,
                           int num_cus, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  switch (kind) {
    case QuantKind::E4M3_1x128: {
      // grid-stride: at most 16 blocks per CU, each block 16 groups per step
      const int64_t groups = rows * (cols / 128);
      int64_t blocks = (groups + 15) / 16;
      const int64_t cap = (int64_t)(num_cus > 0 ? num_cus : 256) * 16;
      if (blocks > cap) blocks = cap;
      dim3 grid((unsigned)blocks);
      trace_launch(kInfoQuantE4m3_1x128, grid, "rows=%lld cols=%lld %s%s", (long long)rows, (long long)cols,
                   bf16 ? "bf16" : "fp32", silu ? " silu_mul" : "");
      if (bf16) {
        if (silu) hipLaunchKernelGGL((quant_e4m3_1x128_kernel<true, true>), grid, dim3(256), 0, st, x, rows, cols, ldx, rows_dev, (uint8_t*)q, (float*)scales);
        else hipLaunchKernelGGL((quant_e4m3_1x128_kernel<true, false>), grid, dim3(256), 0, st, x, rows, cols, ldx, rows_dev, (uint8_t*)q, (float*)scales);
      } else {
        if (silu) hipLaunchKernelGGL((quant_e4m3_1x128_kernel<false, true>), grid, dim3(256), 0, st, x, rows, cols, ldx, rows_dev, (uint8_t*)q, (float*)scales);
        else hipLaunchKernelGGL((quant_e4m3_1x128_kernel<false, false>), grid, dim3(256), 0, st, x, rows, cols, ldx, rows_dev, (uint8_t*)q, (float*)scales);
      }
      break;
    }
    case QuantKind::E4M3_128x128: {
      dim3 grid((unsigned)((rows / 128) * (cols / 128)));
      trace_launch(kInfoQuantE4m3_128x128, grid, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
      if (bf16) hipLaunchKernelGGL((quant_e4m3_128x128_kernel<true>), grid, dim3(256), 0, st, x, rows, cols, ldx, (uint8_t*)q, (float*)scales);
      else hipLaunchKernelGGL((quant_e4m3_128x128_kernel<false>), grid, dim3(256), 0, st, x, rows, cols, ldx, (uint8_t*)q, (float*)scales);
      break;
    }
    case QuantKind::E2M1_1x16: {
      dim3 grid((unsigned)((rows * (cols / 16) + 255) / 256));
      trace_launch(kInfoQuantE2m1_1x16, grid, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
      if (bf16) hipLaunchKernelGGL((quant_e2m1_1x16_kernel<true>), grid, dim3(256), 0, st, x, rows, cols, ldx, (uint8_t*)q, (float*)scales);
      else hipLaunchKernelGGL((quant_e2m1_1x16_kernel<false>), grid, dim3(256), 0, st, x, rows, cols, ldx, (uint8_t*)q, (float*)scales);
      break;
    }
    case QuantKind::E2M1_E8M0_1x32: {
      dim3 grid((unsigned)((rows * (cols / 32) + 255) / 256));
      trace_launch(kInfoQuantE2m1E8m0_1x32, grid, "rows=%lld cols=%lld", (long long)rows, (long long)cols);
      if (bf16) hipLaunchKernelGGL((quant_e2m1_e8m0_1x32_kernel<true>), grid, dim3(256), 0, st, x, rows, cols, ldx, (uint8_t*)q, (uint8_t*)scales);
      else hipLaunchKernelGGL((quant_e2m1_e8m0_1x32_kernel<false>), grid, dim3(256), 0, st, x, rows, cols, ldx, (uint8_t*)q, (uint8_t*)scales);
      break;
    }
  }
  return hipGetLastError();
}

}  // namespace fgg
