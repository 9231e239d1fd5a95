// Masked-layout (decode) grouped GEMM: A is e4m3 [G][M<=16][K] with 1x128
// scales, B is either packed E2M1 with an E8M0 scale per 32 along K, or e4m3
// with 128x128 scales.  Group g computes rows m < masked_m[g] only.
//
//   D[g][m][n] = bf16( Σ_kb sA[g][kb][m] · Σ_{k in kb} A[g][m][k] · B[g][n][k] · 2^(eB[g][n][k/32]-127) )
//
// Decode has M = 1..16 rows per expert, so the kernel is bound by streaming
// the expert weights from HBM ([Infra] "腾讯 AI Infra", Q "量化矩阵乘的维度和
// 流程": weight-only decode has arithmetic intensity 2 / bytes-per-weight;
// [DeepGEMM] bhfrc.com/news/60438 §1.2: decode M is 1..16, MoE segments are
// ragged).  Packed FP4 stays packed into the matrix core and only the fp32
// result is converted ([FP4MoE] "Blackwell架构下FP4 MoE模型的TFLOPS性能优化"
// §3.1 16-byte packed blocks, §4.2 keep FP4 inside the compute).
//
// gfx950 mapping: one v_mfma_scale_f32_16x16x128_f8f6f4 per 128-wide K block
// with the weight tile as the first operand (FP4: 16 contiguous bytes per lane,
// lane group q holding K [32q, 32q+32), its E8M0 scale supplied by the same
// lane) and the activation tile as the second (e4m3: lane group q holds K
// [16q, 16q+16) and [64+16q, 64+16q+16)).  The activation scale sA is fp32, so
// each K block's partial product is promoted with one FMA per output.  Each
// wave owns 16 rows x 16*NT columns and streams its weight rows with 16-byte
// loads, U K blocks per step; the four waves of a workgroup share the
// activation rows through L1.
#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

template <bool B_FP4, int NT, int U>
__global__ void __launch_bounds__(256)
gemm_masked_kernel(int G, int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
                   const float* __restrict__ SA, const uint8_t* __restrict__ B, const void* __restrict__ SBv,
                   const int32_t* __restrict__ masked_m, uint16_t* __restrict__ D, int64_t ldd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t cols_per_wg = 4 * 16 * NT;
  const int64_t wg_per_group = N / cols_per_wg;
  const int g = (int)(blockIdx.x / wg_per_group);
  const int64_t n_base = (blockIdx.x % wg_per_group) * cols_per_wg + wave * 16 * NT;
  int mm = masked_m[g];
  mm = mm < 0 ? 0 : (mm > (int)M ? (int)M : mm);
  if (mm == 0) return;
  const int nkb = (int)(K / 128);
  const bool row_live = l16 < mm;

  const uint8_t* Ag = A + ((int64_t)g * M + l16) * K;
  const float* SAg = SA + (int64_t)g * nkb * M + l16;
  const int64_t kb_bytes = B_FP4 ? 64 : 128;   // bytes of one B row per 128-wide K block
  const uint8_t* Bg = B + ((int64_t)g * N + n_base + l16) * (K * kb_bytes / 128);

  v4f acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int kb0 = 0; kb0 < nkb; kb0 += U) {
    v8i af[U];
    float sa[U];
    v8i bfr[U][NT];
    int bsc[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u;
      const bool kl = kb < nkb;
      if (row_live && kl) {
        const uint4 lo = *reinterpret_cast<const uint4*>(Ag + (int64_t)kb * 128 + 16 * q);
        const uint4 hi = *reinterpret_cast<const uint4*>(Ag + (int64_t)kb * 128 + 64 + 16 * q);
        af[u][0] = (int)lo.x; af[u][1] = (int)lo.y; af[u][2] = (int)lo.z; af[u][3] = (int)lo.w;
        af[u][4] = (int)hi.x; af[u][5] = (int)hi.y; af[u][6] = (int)hi.z; af[u][7] = (int)hi.w;
        sa[u] = SAg[(int64_t)kb * M];
      } else {
        af[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        sa[u] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const uint8_t* brow = Bg + (int64_t)(16 * j) * (K * kb_bytes / 128);
        if (kl) {
          if (B_FP4) {
            const uint4 v = *reinterpret_cast<const uint4*>(brow + (int64_t)kb * 64 + 16 * q);
            bfr[u][j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            const uint8_t* sbr = reinterpret_cast<const uint8_t*>(SBv) + ((int64_t)g * N + n_base + 16 * j + l16) * (K / 32);
            bsc[u][j] = (int)sbr[kb * 4 + q];
          } else {
            const uint4 lo = *reinterpret_cast<const uint4*>(brow + (int64_t)kb * 128 + 16 * q);
            const uint4 hi = *reinterpret_cast<const uint4*>(brow + (int64_t)kb * 128 + 64 + 16 * q);
            bfr[u][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            const float* sbf = reinterpret_cast<const float*>(SBv) + ((int64_t)g * (N / 128) + (n_base + 16 * j) / 128) * nkb;
            bsc[u][j] = __float_as_int(sbf[kb]);
          }
        } else {
          bfr[u][j] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          bsc[u][j] = B_FP4 ? 127 : 0;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        v4f p;
        float s;
        if (B_FP4) {
          p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[u][j], af[u], v4f{0.f, 0.f, 0.f, 0.f}, 4, 0, 0,
                                                                bsc[u][j], 0, 127);
          s = sa[u];
        } else {
          p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[u][j], af[u], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                127, 0, 127);
          s = sa[u] * __int_as_float(bsc[u][j]);
        }
        acc[j][0] = fmaf(p[0], s, acc[j][0]);
        acc[j][1] = fmaf(p[1], s, acc[j][1]);
        acc[j][2] = fmaf(p[2], s, acc[j][2]);
        acc[j][3] = fmaf(p[3], s, acc[j][3]);
      }
    }
  }
  if (!row_live) return;
  uint16_t* drow = D + ((int64_t)g * M + l16) * ldd + n_base + 4 * q;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const uint32_t lo = (uint32_t)bf16_bits_rne(acc[j][0]) | ((uint32_t)bf16_bits_rne(acc[j][1]) << 16);
    const uint32_t hi = (uint32_t)bf16_bits_rne(acc[j][2]) | ((uint32_t)bf16_bits_rne(acc[j][3]) << 16);
    *reinterpret_cast<uint2*>(drow + 16 * j) = make_uint2(lo, hi);
  }
}

hipError_t launch_gemm_masked(bool b_fp4, int32_t G, int64_t M, int64_t N, int64_t K,
                              const uint8_t* a, const float* sa, const uint8_t* b, const void* sb,
                              const int32_t* masked_m, uint16_t* d, int64_t ldd, hipStream_t st) {
  constexpr int NT = 2, U = 4;
  const int64_t cols_per_wg = 4 * 16 * NT;
  if (N % cols_per_wg != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)(G * (N / cols_per_wg)));
  if (b_fp4)
    hipLaunchKernelGGL((gemm_masked_kernel<true, NT, U>), grid, dim3(256), 0, st, G, M, N, K, a, sa, b, sb, masked_m, d, ldd);
  else
    hipLaunchKernelGGL((gemm_masked_kernel<false, NT, U>), grid, dim3(256), 0, st, G, M, N, K, a, sa, b, sb, masked_m, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
