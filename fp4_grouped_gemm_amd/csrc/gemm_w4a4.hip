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
// small bf16-MFMA kernel for T = X·L_down (fp32 accumulate, stored bf16 in
// the workspace, with L_down transposed there first) and one extra bf16 MFMA
// step T·L_up per output tile, before the bias is added in the epilogue.
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

// L_down [K][32] -> LdT [32][K] (bf16), so that both operands of T = X·L_down
// are K-contiguous.
__global__ void __launch_bounds__(256) w4a4_ld_transpose_kernel(const uint16_t* __restrict__ Ld, int64_t K,
                                                                uint16_t* __restrict__ LdT) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over K*32, rank fastest (coalesced reads)
  if (i >= K * 32) return;
  const int64_t k = i >> 5, r = i & 31;
  LdT[r * K + k] = Ld[i];
}

// T[m][r] = Σ_k X[m][k] · L_down[k][r] (rank 32), fp32 accumulate, stored bf16.
// One 256-thread block per 16 rows; wave w sums K range [w·K/4, (w+1)·K/4) with
// v_mfma_f32_16x16x32_bf16 (first operand: 16 ranks of LdT, second: the 16 X
// rows; lane (l, q) holds K elements [8q, 8q+8) of row l of each), two rank
// tiles per wave; the four partial sums are added in wave order through LDS.
__global__ void __launch_bounds__(256) w4a4_lowrank_down_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                                 const uint16_t* __restrict__ LdT,
                                                                 uint16_t* __restrict__ T) {
  __shared__ v4f part[4][2][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  int64_t mrow = m0 + l16;
  if (mrow >= M) mrow = M - 1;               // rows past the end read a valid row; never stored
  const int64_t kq = K / 4;                  // K % 128 == 0, so kq % 32 == 0
  const int64_t k_begin = wave * kq, k_end = k_begin + kq;
  const uint16_t* xr = X + mrow * K + 8 * q;
  const uint16_t* l0 = LdT + (int64_t)l16 * K + 8 * q;
  const uint16_t* l1 = LdT + (int64_t)(16 + l16) * K + 8 * q;
  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
  for (int64_t k = k_begin; k < k_end; k += 128) {
    uint4 xa[4], la[4], lb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (k + 32 * u >= k_end) break;       // wave-uniform: the range is a multiple of 32
      xa[u] = *reinterpret_cast<const uint4*>(xr + k + 32 * u);
      la[u] = *reinterpret_cast<const uint4*>(l0 + k + 32 * u);
      lb[u] = *reinterpret_cast<const uint4*>(l1 + k + 32 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (k + 32 * u >= k_end) break;
      const v8bf xv = __builtin_bit_cast(v8bf, xa[u]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, la[u]), xv, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, lb[u]), xv, acc1, 0, 0, 0);
    }
  }
  part[wave][0][lane] = acc0;
  part[wave][1][lane] = acc1;
  __syncthreads();
  if (wave != 0) return;
  // lane (l16, q) holds ranks 4q..4q+3 (tile 0) and 16+4q.. (tile 1) of row m0 + l16
  v4f s0 = part[0][0][lane], s1 = part[0][1][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const v4f a = part[w][0][lane], b = part[w][1][lane];
    s0[0] += a[0]; s0[1] += a[1]; s0[2] += a[2]; s0[3] += a[3];
    s1[0] += b[0]; s1[1] += b[1]; s1[2] += b[2]; s1[3] += b[3];
  }
  const int64_t m = m0 + l16;
  if (m >= M) return;
  uint16_t* t = T + m * 32 + 4 * q;
  *reinterpret_cast<uint2*>(t) = make_uint2((uint32_t)bf16_bits_rne(s0[0]) | ((uint32_t)bf16_bits_rne(s0[1]) << 16),
                                            (uint32_t)bf16_bits_rne(s0[2]) | ((uint32_t)bf16_bits_rne(s0[3]) << 16));
  *reinterpret_cast<uint2*>(t + 16) = make_uint2((uint32_t)bf16_bits_rne(s1[0]) | ((uint32_t)bf16_bits_rne(s1[1]) << 16),
                                                 (uint32_t)bf16_bits_rne(s1[2]) | ((uint32_t)bf16_bits_rne(s1[3]) << 16));
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

// workspace: T [M][32] bf16, then LdT [32][K] bf16 (16-byte aligned)
size_t w4a4_workspace_bytes(int64_t M, int64_t K, int32_t rank) {
  if (rank == 0) return 0;
  return (size_t)(((M * 32 * 2 + 15) / 16) * 16 + 32 * K * 2);
}

hipError_t launch_w4a4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                       const uint8_t* b, const float* sb, const uint16_t* x_bf16,
                       const uint16_t* l_down, const uint16_t* l_up, int32_t rank,
                       const uint16_t* bias, uint16_t* d, int64_t ldd, void* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  uint16_t* T = reinterpret_cast<uint16_t*>(ws);
  if (rank > 0) {
    uint16_t* LdT = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(ws) + ((M * 32 * 2 + 15) / 16) * 16);
    hipLaunchKernelGGL(w4a4_ld_transpose_kernel, dim3((unsigned)((K * 32 + 255) / 256)), dim3(256), 0, st, l_down, K,
                       LdT);
    hipLaunchKernelGGL(w4a4_lowrank_down_kernel, dim3((unsigned)((M + 15) / 16)), dim3(256), 0, st, x_bf16, M, K,
                       LdT, T);
  }
  const int64_t tiles = (M / BM) * (N / BN);
  hipLaunchKernelGGL(w4a4_gemm_kernel, dim3((unsigned)tiles), dim3(256), 0, st, M, N, K, a, sa, b, sb,
                     rank > 0 ? T : nullptr, l_up, (int)rank, bias, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
