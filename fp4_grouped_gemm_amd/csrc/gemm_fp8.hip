// Block-scaled FP8 x FP8 grouped GEMM, contiguous (prefill) layout; the dense
// GEMM is the one-group case.
//
//   D[r][n] = bf16( Σ_kb sA[kb][r] · sB[g][n/128][kb] · Σ_{k in kb} A[r][k] · B[g][n][k] )
//
// The per-group K-block formula is the grouped-K GEMM of [Infra] "腾讯 AI
// Infra", Q "量化矩阵乘的维度和流程", with the activation's per-token group
// scale as well; the scales are applied inside the K loop and the sum is kept
// in fp32 over all of K ([DeepGEMM] bhfrc.com/news/60438 §2.2, §2.3).
//
// gfx950 mapping:
//  * one v_mfma_scale_f32_16x16x128_f8f6f4 covers exactly one 128-wide K block,
//    so the block's partial product comes out of the matrix core on its own
//    (zero accumulator input) and is promoted with one FMA per output element:
//    acc += p · (sA · sB).  The E8M0 operand scales are fixed at 2^0.
//  * the weight tile is the MFMA's first operand, so every lane's four outputs
//    are four consecutive columns of one row: one sA per lane per 16-row
//    subtile, one sB per tile, and 8-byte bf16 stores.
//  * 128 x 128 output tile per 256-thread workgroup (4 waves, each 64 x 64 =
//    4 x 4 MFMA subtiles); A, B and sA K-block tiles are double-buffered in
//    LDS (2 x 32.5 KB), so two workgroups fit one CU.
//  * LDS rows are 128 B; the 16-byte chunk c of row r lives at chunk
//    c ^ ((r ^ (r >> 3)) & 7), which keeps both the row-contiguous tile writes
//    and the 16-row operand reads free of bank conflicts for 32 and 64 banks.
//  * persistent grid: each workgroup strides over the output tiles; a tile's
//    expert is found by binary search over the segment offsets (segments are
//    multiples of 128 rows, so a tile never straddles two experts).
#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kThreads = 256;
constexpr int kStageBytes = BM * BK + BN * BK + BM * 4;   // A + B + sA

__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ inline v8i read_frag(const uint8_t* tile, int row, int q) {
  const uint4* base = reinterpret_cast<const uint4*>(tile + row * BK);
  const int key = swz(row);
  const uint4 lo = base[(2 * q) ^ key];
  const uint4 hi = base[(2 * q + 1) ^ key];
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ inline int find_group(const int32_t* __restrict__ offsets, int G, int64_t row) {
  int lo = 0, hi = G - 1;           // largest g with offsets[g] <= row
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)offsets[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace

__global__ void __launch_bounds__(kThreads, 2)
gemm_fp8_contig_kernel(int G, int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
                       const float* __restrict__ SA, const uint8_t* __restrict__ B,
                       const float* __restrict__ SB, const int32_t* __restrict__ offsets,
                       uint16_t* __restrict__ D, int64_t ldd) {
  __shared__ __align__(16) uint8_t smem[2 * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int l16 = lane & 15, q = lane >> 4;

  const int64_t m_end = offsets ? (int64_t)offsets[G] : M;
  const int64_t m_tiles = (m_end + BM - 1) / BM;
  const int64_t n_tiles = N / BN;
  const int64_t num_tiles = m_tiles * n_tiles;
  const int nkb = (int)(K / BK);
  const int64_t nblk = N / 128;

  // global->LDS copy assignment: thread t moves 16-byte chunk (t % 8) of rows t/8 + 32i
  const int cp_chunk = tid & 7;
  const int cp_row0 = tid >> 3;

  for (int64_t tile = blockIdx.x; tile < num_tiles; tile += gridDim.x) {
    // group 8 M-tiles together, N fastest within the group (operand reuse in L2)
    const int64_t group_span = 8 * n_tiles;
    const int64_t grp = tile / group_span;
    const int64_t first_mt = grp * 8;
    const int64_t gm = (m_tiles - first_mt) < 8 ? (m_tiles - first_mt) : 8;
    const int64_t within = tile - grp * group_span;
    const int64_t mt = first_mt + within % gm;
    const int64_t nt = within / gm;
    const int64_t m0 = mt * BM, n0 = nt * BN;
    const int g = offsets ? find_group(offsets, G, m0) : 0;
    const uint8_t* Bg = B + ((int64_t)g * N + n0) * K;
    const float* SBg = SB + ((int64_t)g * nblk + n0 / 128) * nkb;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint4 ra[4], rb[4];
    float rsa = 0.f;
    auto gload = [&](int kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = cp_row0 + 32 * i;
        const int64_t grow = m0 + r;
        if (grow < m_end)
          ra[i] = *reinterpret_cast<const uint4*>(A + grow * K + (int64_t)kb * BK + cp_chunk * 16);
        else
          ra[i] = make_uint4(0, 0, 0, 0);
        rb[i] = *reinterpret_cast<const uint4*>(Bg + (int64_t)r * K + (int64_t)kb * BK + cp_chunk * 16);
      }
      if (tid < BM) rsa = (m0 + tid < m_end) ? SA[(int64_t)kb * M + m0 + tid] : 0.0f;
    };
    auto lstore = [&](int stage) {
      uint8_t* sa_t = smem + stage * kStageBytes;
      uint8_t* sb_t = sa_t + BM * BK;
      float* ss_t = reinterpret_cast<float*>(sb_t + BN * BK);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = cp_row0 + 32 * i;
        const int pc = cp_chunk ^ swz(r);
        *reinterpret_cast<uint4*>(sa_t + r * BK + pc * 16) = ra[i];
        *reinterpret_cast<uint4*>(sb_t + r * BK + pc * 16) = rb[i];
      }
      if (tid < BM) ss_t[tid] = rsa;
    };

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
      const int stage = kb & 1;
      if (kb + 1 < nkb) gload(kb + 1);
      const uint8_t* sa_t = smem + stage * kStageBytes;
      const uint8_t* sb_t = sa_t + BM * BK;
      const float* ss_t = reinterpret_cast<const float*>(sb_t + BN * BK);
      const float sb = SBg[kb];

      v8i af[4], bf[4];
      float sab[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = read_frag(sa_t, wm * 64 + 16 * i + l16, q);
        sab[i] = ss_t[wm * 64 + 16 * i + l16] * sb;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = read_frag(sb_t, wn * 64 + 16 * j + l16, q);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bf[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
          acc[i][j][0] = fmaf(p[0], sab[i], acc[i][j][0]);
          acc[i][j][1] = fmaf(p[1], sab[i], acc[i][j][1]);
          acc[i][j][2] = fmaf(p[2], sab[i], acc[i][j][2]);
          acc[i][j][3] = fmaf(p[3], sab[i], acc[i][j][3]);
        }
      }
      if (kb + 1 < nkb) lstore(stage ^ 1);
      __syncthreads();
    }

    // epilogue: lane holds columns n0 + wn*64 + 16j + 4q + (0..3) of row m0 + wm*64 + 16i + l16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + wm * 64 + 16 * i + l16;
      if (row >= m_end) continue;
      uint16_t* drow = D + row * ldd + n0 + wn * 64 + 4 * q;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (uint32_t)bf16_bits_rne(acc[i][j][0]) | ((uint32_t)bf16_bits_rne(acc[i][j][1]) << 16);
        const uint32_t hi = (uint32_t)bf16_bits_rne(acc[i][j][2]) | ((uint32_t)bf16_bits_rne(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(drow + 16 * j) = make_uint2(lo, hi);
      }
    }
  }
}

hipError_t launch_gemm_fp8_contig(int32_t G, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                  const float* sa, const uint8_t* b, const float* sb,
                                  const int32_t* offsets, uint16_t* d, int64_t ldd, int num_cus,
                                  hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles_upper = ((M + BM - 1) / BM) * (N / BN);
  int64_t grid = (int64_t)num_cus * 2;
  if (grid > tiles_upper) grid = tiles_upper;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(gemm_fp8_contig_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, G, M,
                     N, K, a, sa, b, sb, offsets, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
