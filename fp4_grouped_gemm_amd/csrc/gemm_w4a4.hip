// W4A4 GEMM with a low-rank residual and a per-column bias:
//   Y = (Q(X) · Q(W)ᵀ) ⊙ scale + L(X) + b,     L(X) = (X · L_down) · L_up
// ([W4A4] "最新GPU架构上W4A4算子的Warp专用化内核实践" §1, operator equation).
// Q(X), Q(W) are E2M1 with one fp32 scale per 16 elements along K, and ⊙ scale
// applies the pair of group scales to each 16-element partial sum.
//
// gfx950 has no matrix instruction that applies an arbitrary fp32 scale per 16
// elements, and promoting 16-wide partial sums on the vector ALU would cost
// M·N·K/16 FMAs (more than the matrix work).  So each operand tile is
// dequantized once on its way into LDS, x·s rounded to fp16, and contracted
// with v_mfma_f32_16x16x32_f16 in fp32.  The low-rank branch is a separate
// small kernel for T = X·L_down (fp32 accumulate, stored bf16 in the
// workspace) and one extra bf16 MFMA step T·L_up per output tile, before the
// bias is added in the epilogue.
//
// Tile: 128 x 128 per 256-thread workgroup (4 waves of 64 x 64); one 128-wide
// K block per LDS stage (2 x 128 x 128 fp16 = 64 KB); 16-byte chunks of each
// 256-byte LDS row are XOR-swizzled by the row index.
#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {
constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kRowBytes = BK * 2;   // fp16 row in LDS

__device__ inline float e2m1_f32(uint32_t nib, float s) {
  const uint32_t mag = nib & 7u;
  float f = __uint_as_float((mag + 252u) << 22);        // exact for magnitude codes >= 2
  f = (mag < 2u) ? 0.5f * (float)mag : f;              // 0 and 0.5
  f = (nib & 8u) ? -f : f;
  return f * s;
}

// dequantize 32 packed E2M1 values (16 bytes, two 16-element groups) to fp16
__device__ inline void dequant32(uint4 packed, float s0, float s1, uint4* out4) {
  const uint32_t w[4] = {packed.x, packed.y, packed.z, packed.w};
  uint32_t h[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float s = (i < 2) ? s0 : s1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (w[i] >> (8 * j)) & 0xFFu;
      const _Float16 lo = (_Float16)e2m1_f32(byte & 0xFu, s);
      const _Float16 hi = (_Float16)e2m1_f32(byte >> 4, s);
      h[4 * i + j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
  }
  out4[0] = make_uint4(h[0], h[1], h[2], h[3]);
  out4[1] = make_uint4(h[4], h[5], h[6], h[7]);
  out4[2] = make_uint4(h[8], h[9], h[10], h[11]);
  out4[3] = make_uint4(h[12], h[13], h[14], h[15]);
}

__device__ inline int swz16(int row) { return row & 15; }
}  // namespace

// T[m][r] = Σ_k X[m][k] · L_down[k][r] in fp32, stored bf16.  8 rows x 32 ranks per block.
__global__ void __launch_bounds__(256) w4a4_lowrank_down_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                                 const uint16_t* __restrict__ Ld, int rank,
                                                                 uint16_t* __restrict__ T) {
  __shared__ float xs[8][256];
  __shared__ float ls[256][33];
  const int r = threadIdx.x & 31, i = threadIdx.x >> 5;
  const int64_t m = (int64_t)blockIdx.x * 8 + i;
  float acc = 0.0f;
  for (int64_t k0 = 0; k0 < K; k0 += 256) {
    for (int idx = threadIdx.x; idx < 8 * 256; idx += 256) {
      const int ii = idx >> 8, kk = idx & 255;
      const int64_t mm = (int64_t)blockIdx.x * 8 + ii;
      xs[ii][kk] = (mm < M && k0 + kk < K) ? bf16_to_f32(X[mm * K + k0 + kk]) : 0.0f;
    }
    for (int idx = threadIdx.x; idx < 256 * 32; idx += 256) {
      const int kk = idx >> 5, rr = idx & 31;
      ls[kk][rr] = (k0 + kk < K && rr < rank) ? bf16_to_f32(Ld[(k0 + kk) * rank + rr]) : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 256; ++kk) acc = fmaf(xs[i][kk], ls[kk][r], acc);
    __syncthreads();
  }
  if (m < M && r < rank) T[m * rank + r] = bf16_bits_rne(acc);
}

__global__ void __launch_bounds__(256, 1)
w4a4_gemm_kernel(int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A, const float* __restrict__ SA,
                 const uint8_t* __restrict__ B, const float* __restrict__ SB,
                 const uint16_t* __restrict__ T, const uint16_t* __restrict__ Lu, int rank,
                 const uint16_t* __restrict__ bias, uint16_t* __restrict__ D, int64_t ldd) {
  __shared__ __align__(16) uint8_t smem[2 * BM * kRowBytes];   // A tile then B tile, fp16
  uint8_t* at = smem;
  uint8_t* bt = smem + BM * kRowBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t n_tiles = N / BN;
  const int64_t m0 = (blockIdx.x / n_tiles) * BM, n0 = (blockIdx.x % n_tiles) * BN;
  const int64_t ng = K / 16;
  const int nkb = (int)(K / BK);

  // copy assignment: 128 rows x 4 chunks of 32 elements; thread t: chunk t%4, rows t/4 + 64i
  const int cc = tid & 3, cr0 = tid >> 2;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 pa[2], pb[2];
  float2 sa2[2], sb2[2];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t ra = m0 + cr0 + 64 * i, rb = n0 + cr0 + 64 * i;
      pa[i] = *reinterpret_cast<const uint4*>(A + ra * (K / 2) + (int64_t)kb * 64 + cc * 16);
      pb[i] = *reinterpret_cast<const uint4*>(B + rb * (K / 2) + (int64_t)kb * 64 + cc * 16);
      sa2[i] = *reinterpret_cast<const float2*>(SA + ra * ng + (int64_t)kb * 8 + cc * 2);
      sb2[i] = *reinterpret_cast<const float2*>(SB + rb * ng + (int64_t)kb * 8 + cc * 2);
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = cr0 + 64 * i;
      uint4 h[4];
      dequant32(pa[i], sa2[i].x, sa2[i].y, h);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4*>(at + r * kRowBytes + (((cc * 4 + c) ^ swz16(r)) * 16)) = h[c];
      dequant32(pb[i], sb2[i].x, sb2[i].y, h);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint4*>(bt + r * kRowBytes + (((cc * 4 + c) ^ swz16(r)) * 16)) = h[c];
    }
  };

  gload(0);
  for (int kb = 0; kb < nkb; ++kb) {
    __syncthreads();           // previous step's LDS reads are done
    lstore();
    __syncthreads();
    if (kb + 1 < nkb) gload(kb + 1);
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      v8h af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + 16 * i + l16;
        const uint4 v = *reinterpret_cast<const uint4*>(at + r * kRowBytes + (((s * 4 + q) ^ swz16(r)) * 16));
        af[i] = __builtin_bit_cast(v8h, v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + 16 * j + l16;
        const uint4 v = *reinterpret_cast<const uint4*>(bt + r * kRowBytes + (((s * 4 + q) ^ swz16(r)) * 16));
        bf[j] = __builtin_bit_cast(v8h, v);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // low-rank step: acc += T[m][0:32] · L_up[0:32][n]  (one bf16 MFMA K step of 32)
  if (rank == 32) {
    v8bf tf[4], lf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 64 + 16 * i + l16;
      tf[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(T + m * 32 + 8 * q));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + 16 * j + l16;
      uint16_t u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = Lu[(int64_t)(8 * q + e) * N + n];
      lf[j] = __builtin_bit_cast(v8bf, u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lf[j], tf[i], acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + wm * 64 + 16 * i + l16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + wn * 64 + 16 * j + 4 * q;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32(bias[n + e]);
      }
      const uint32_t lo = (uint32_t)bf16_bits_rne(v[0]) | ((uint32_t)bf16_bits_rne(v[1]) << 16);
      const uint32_t hi = (uint32_t)bf16_bits_rne(v[2]) | ((uint32_t)bf16_bits_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(D + row * ldd + n) = make_uint2(lo, hi);
    }
  }
}

size_t w4a4_workspace_bytes(int64_t M, int32_t rank) { return (size_t)(M * rank * 2); }

hipError_t launch_w4a4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                       const uint8_t* b, const float* sb, const uint16_t* x_bf16,
                       const uint16_t* l_down, const uint16_t* l_up, int32_t rank,
                       const uint16_t* bias, uint16_t* d, int64_t ldd, void* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  uint16_t* T = reinterpret_cast<uint16_t*>(ws);
  if (rank > 0) {
    hipLaunchKernelGGL(w4a4_lowrank_down_kernel, dim3((unsigned)((M + 7) / 8)), dim3(256), 0, st, x_bf16, M, K,
                       l_down, (int)rank, T);
  }
  const int64_t tiles = (M / BM) * (N / BN);
  hipLaunchKernelGGL(w4a4_gemm_kernel, dim3((unsigned)tiles), dim3(256), 0, st, M, N, K, a, sa, b, sb,
                     rank > 0 ? T : nullptr, l_up, (int)rank, bias, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
