// W4A4 GEMM with a low-rank residual and a per-column bias:
//   Y = (Q(X) · Q(W)ᵀ) ⊙ scale + L(X) + b,     L(X) = (X · L_down) · L_up
// ([W4A4] "最新GPU架构上W4A4算子的Warp专用化内核实践" §1, operator equation).
// Q(X), Q(W) are E2M1 with one fp32 scale per 16 elements along K, and ⊙ scale
// applies the pair of group scales to each 16-element partial sum.
//
// gfx950 has no matrix instruction that applies an arbitrary fp32 scale per 16
// elements, and promoting 16-wide partial sums on the vector ALU would cost
// M·N·K/16 FMAs (more than the matrix work).  So each operand is dequantized
// once, x·s rounded to fp16, into the workspace (w4a4_prep_kernel: every
// element exactly once; dequantizing inside the GEMM made each workgroup redo
// the tiles it shares with N/128 or M/128 others and left the kernel bound by
// that vector-ALU work), and contracted with v_mfma_f32_16x16x32_f16 in fp32.
// The low-rank branch is a separate small bf16-MFMA kernel for T = X·L_down
// (fp32 accumulate, stored bf16 in the workspace, with L_down transposed there
// first) and one extra bf16 MFMA step T·L_up per output tile, before the bias
// is added in the epilogue.
//
// GEMM tile: 128 x 128 per 512-thread workgroup: 8 waves, each a 64 x 64 quadrant
// and one of the two 32-wide halves of every K stage (two waves per SIMD; the two
// halves' fp32 sums are added through LDS at the end); a 4-buffer LDS ring of
// 64-wide K stages (A and B, 2 x 128 rows x 128 bytes of fp16 = 32 KB each)
// filled by global_load_lds_dwordx4 with up to three stages in flight, the next
// stage's fragments read into registers while the current stage's MFMAs run; each
// 128-byte row's 16-byte chunks XOR-swizzled by the row index.
#include <algorithm>
#include <type_traits>

#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {
constexpr int BM = 128, BN = 128;
constexpr int BKH = 64;                       // K elements per LDS stage
constexpr int kRowBytes = BKH * 2;            // one fp16 row of a stage: 128 bytes
constexpr int kTileBytes = BM * kRowBytes;    // 16 KB (A or B)
constexpr int kStageBytes = 2 * kTileBytes;   // A then B
constexpr int kStages = 4;
constexpr int kWaves = 8;                     // 2 x 2 output quadrants x 2 halves of each K stage
constexpr int kDmaPerStage = kStageBytes / 1024 / kWaves;   // 1 KB DMA instructions per wave per stage

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

// 16-byte chunk swizzle of a 128-byte row (as in the FP8 GEMM): rows 16 apart share a
// key; any 8 consecutive rows get 8 distinct keys
__device__ inline int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

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

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
}  // namespace

// The GEMM's operand preparation in one launch, by block ranges: packed E2M1 rows with
// fp32 scales per 16 -> fp16 (x·s rounded once), for A ([M][K/2] -> [M][K]) and B,
// one thread per 32 elements; then, with the low-rank branch, L_down [K][32] ->
// LdT [32][K] (bf16), so that both operands of T = X·L_down are K-contiguous.
__device__ inline void dequant_item(const uint8_t* __restrict__ q, const float* __restrict__ s, int64_t i,
                                    uint16_t* __restrict__ out) {
  const uint4 p = *reinterpret_cast<const uint4*>(q + i * 16);
  const float2 sc = *reinterpret_cast<const float2*>(s + i * 2);
  uint4 h[4];
  dequant32(p, sc.x, sc.y, h);
  uint4* o = reinterpret_cast<uint4*>(out + i * 32);
  o[0] = h[0];
  o[1] = h[1];
  o[2] = h[2];
  o[3] = h[3];
}

__global__ void __launch_bounds__(256) w4a4_prep_kernel(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                        int64_t na, uint16_t* __restrict__ ah,
                                                        const uint8_t* __restrict__ qb, const float* __restrict__ sb,
                                                        int64_t nb, uint16_t* __restrict__ bh,
                                                        const uint16_t* __restrict__ Ld, int64_t nld,
                                                        uint16_t* __restrict__ LdT, int64_t K) {
  const int64_t ba = (na + 255) / 256, bb = (nb + 255) / 256;
  const int64_t blk = blockIdx.x;
  if (blk < ba) {
    const int64_t i = blk * 256 + threadIdx.x;
    if (i < na) dequant_item(qa, sa, i, ah);
  } else if (blk < ba + bb) {
    const int64_t i = (blk - ba) * 256 + threadIdx.x;
    if (i < nb) dequant_item(qb, sb, i, bh);
  } else {
    const int64_t i = (blk - ba - bb) * 256 + threadIdx.x;   // over K*32, rank fastest (coalesced reads)
    if (i < nld) LdT[(i & 31) * K + (i >> 5)] = Ld[i];
  }
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

__global__ void __launch_bounds__(512, 1)
w4a4_gemm_kernel(int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ Ah, const uint16_t* __restrict__ Bh,
                 const uint16_t* __restrict__ T, const uint16_t* __restrict__ Lu, int rank,
                 const uint16_t* __restrict__ bias, uint16_t* __restrict__ D, int64_t ldd) {
  __shared__ __align__(16) uint8_t smem[kStages * kStageBytes];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = (wave >> 1) & 1, kw = wave >> 2;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t n_tiles = N / BN;
  const int64_t m0 = (blockIdx.x / n_tiles) * BM, n0 = (blockIdx.x % n_tiles) * BN;
  const int nks = (int)(K / BKH);

  // DMA roles: a stage is 32 segments of 1 KB (8 rows of 128 bytes): segments 0-15 the A
  // rows, 16-31 the B rows; wave w issues segments 4w .. 4w+3.  Lane l fills chunk l % 8 of
  // row l / 8 of its segment and reads source chunk (l % 8) ^ swz(row).
  const int lrow = lane >> 3;
  const uint8_t* Abase = reinterpret_cast<const uint8_t*>(Ah + m0 * K);
  const uint8_t* Bbase = reinterpret_cast<const uint8_t*>(Bh + n0 * K);
  uint32_t voff[kDmaPerStage];
#pragma unroll
  for (int i = 0; i < kDmaPerStage; ++i) {
    const int seg = (wave * kDmaPerStage + i) & 15;
    const int row = seg * 8 + lrow;
    voff[i] = (uint32_t)row * (uint32_t)(K * 2) + (uint32_t)((((lane & 7) ^ swz(row))) * 16);
  }
  auto issue = [&](int ks, int stage) {
    const uint8_t* src = (wave < kWaves / 2 ? Abase : Bbase) + (int64_t)ks * (BKH * 2);
#pragma unroll
    for (int i = 0; i < kDmaPerStage; ++i)
      dma16(src, voff[i], lds_base + stage * kStageBytes + (wave * kDmaPerStage + i) * 1024);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // fragment reads: lane (l16, q) takes 8 fp16 (K [8q, 8q+8) of the wave's 32-K half kw
  // of a stage) of rows 16 i + l16 of its A rows and of its B rows; rows 16 apart share a
  // swizzle key, so each fragment is a lane base plus an immediate
  const int arow = wm * 64 + l16, brow = wn * 64 + l16;
  const int a_off = arow * kRowBytes + (((4 * kw + q) ^ swz(arow)) << 4);
  const int b_off = brow * kRowBytes + (((4 * kw + q) ^ swz(brow)) << 4);
  // One stage: the MFMAs of stage ks run on fragments already in registers while the
  // fragments of stage ks + 1 are read from LDS (two register sets in rotation).
  //   top of step ks: this wave's DMA of stage ks + 1 done (the groups of stages ks + 2,
  //   ks + 3 may fly), its reads of stage ks done; the barrier makes both true for every
  //   wave, so buffer ks % 4 is free and takes stage ks + 4.
  struct Frags {
    v8h a[4], b[4];
  };
  auto read_frags = [&](int slot, Frags& f) {
    const uint8_t* at = smem + slot * kStageBytes + a_off;
    const uint8_t* bt = smem + slot * kStageBytes + kTileBytes + b_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const v8h*>(at + 16 * i * kRowBytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = *reinterpret_cast<const v8h*>(bt + 16 * j * kRowBytes);
  };
  auto step = [&](auto st_tag, int ks, const Frags& cur, Frags& nxt) {
    constexpr int ST = decltype(st_tag)::value;     // == ks % 4
    const int after = nks - 2 - ks;                 // stages issued after stage ks + 1
    if (after >= 2) wait_vmcnt<2 * kDmaPerStage>();
    else if (after == 1) wait_vmcnt<kDmaPerStage>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (ks + 4 < nks) issue(ks + 4, ST);
    if (ks + 1 < nks) read_frags((ST + 1) % kStages, nxt);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.b[j], cur.a[i], acc[i][j], 0, 0, 0);
  };
  if (nks > 0) issue(0, 0);
  if (nks > 1) issue(1, 1);
  if (nks > 2) issue(2, 2);
  if (nks > 3) issue(3, 3);
  // stage 0 landed (three groups may fly)
  if (nks > 3) wait_vmcnt<3 * kDmaPerStage>();
  else if (nks > 2) wait_vmcnt<2 * kDmaPerStage>();
  else if (nks > 1) wait_vmcnt<kDmaPerStage>();
  else wait_vmcnt<0>();
  __syncthreads();
  Frags f0, f1;
  if (nks > 0) read_frags(0, f0);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  for (int ks = 0; ks < nks; ks += 4) {
    step(I0{}, ks, f0, f1);
    if (ks + 1 < nks) step(I1{}, ks + 1, f1, f0);
    if (ks + 2 < nks) step(I2{}, ks + 2, f0, f1);
    if (ks + 3 < nks) step(I3{}, ks + 3, f1, f0);
  }

  // the two K halves: waves 4-7 hand their sums to waves 0-3 through the (now free) ring
  __syncthreads();
  v4f* red = reinterpret_cast<v4f*>(smem);        // [4 quadrants][16 subtiles][64 lanes]
  if (kw == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[((wave & 3) * 16 + 4 * i + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  if (kw == 1) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v4f o = red[((wave & 3) * 16 + 4 * i + j) * 64 + lane];
      acc[i][j][0] += o[0];
      acc[i][j][1] += o[1];
      acc[i][j][2] += o[2];
      acc[i][j][3] += o[3];
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

// workspace: A and B dequantized to fp16 ([M][K], [N][K]), then with the low-rank
// branch T [M][32] bf16 and LdT [32][K] bf16; every part 256-byte aligned
namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

size_t w4a4_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank) {
  size_t b = align256((size_t)M * K * 2) + align256((size_t)N * K * 2);
  if (rank > 0) b += align256((size_t)M * 32 * 2) + align256((size_t)32 * K * 2);
  return b;
}

hipError_t launch_w4a4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                       const uint8_t* b, const float* sb, const uint16_t* x_bf16,
                       const uint16_t* l_down, const uint16_t* l_up, int32_t rank,
                       const uint16_t* bias, uint16_t* d, int64_t ldd, void* ws, int num_cus, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M % BM != 0 || N % BN != 0 || K % 128 != 0 || K == 0) return hipErrorInvalidValue;
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  uint16_t* Ah = reinterpret_cast<uint16_t*>(w);
  uint16_t* Bh = reinterpret_cast<uint16_t*>(w + align256((size_t)M * K * 2));
  uint8_t* rest = w + align256((size_t)M * K * 2) + align256((size_t)N * K * 2);
  (void)num_cus;
  const int64_t na = M * K / 32, nb = N * K / 32, nld = rank > 0 ? K * 32 : 0;
  uint16_t* T = reinterpret_cast<uint16_t*>(rest);
  uint16_t* LdT = reinterpret_cast<uint16_t*>(rest + align256((size_t)M * 32 * 2));
  const int64_t blocks = (na + 255) / 256 + (nb + 255) / 256 + (nld + 255) / 256;
  hipLaunchKernelGGL(w4a4_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, sa, na, Ah, b, sb, nb, Bh,
                     l_down, nld, rank > 0 ? LdT : nullptr, K);
  if (rank > 0)
    hipLaunchKernelGGL(w4a4_lowrank_down_kernel, dim3((unsigned)((M + 15) / 16)), dim3(256), 0, st, x_bf16, M, K,
                       LdT, T);
  const int64_t tiles = (M / BM) * (N / BN);
  hipLaunchKernelGGL(w4a4_gemm_kernel, dim3((unsigned)tiles), dim3(64 * kWaves), 0, st, M, N, K, Ah, Bh,
                     rank > 0 ? T : nullptr, l_up, (int)rank, bias, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
