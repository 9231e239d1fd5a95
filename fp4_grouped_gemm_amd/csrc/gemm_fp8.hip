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
//    subtile, one sB per wave (a wave's 64 columns lie in one 128-column scale
//    block), and 8-byte bf16 stores.
//  * workgroup tile 128 x 256: 8 waves of 64 x 64 (4 x 4 MFMA subtiles, 64 fp32
//    accumulators per lane), two waves per SIMD so that one wave's MFMAs
//    overlap the other's promotion FMAs, LDS reads and barrier waits; one
//    workgroup per CU.
//  * a 3-stage LDS ring (3 x 48.5 KB) filled by global_load_lds_dwordx4, the
//    gfx950 direct global->LDS path: no register staging, two K blocks in
//    flight while the third is consumed ([FP4MoE] §3.2 double-buffered
//    pipeline; [W4A4] §5 stage index/phase discipline, here a fixed rotation
//    kb % 3).  The LDS writes are issued from inline asm and their completion
//    is counted by hand with s_waitcnt vmcnt, because the compiler's own wait
//    insertion cannot tell which stage a read depends on and would drain the
//    whole ring before every read.  No other vector-memory instruction is
//    issued inside the K loop (scale sB comes through the scalar cache), so
//    each wave's vmcnt counts exactly its own DMA instructions.
//  * LDS rows are 128 B; the 16-byte chunk c of row r lives at chunk
//    c ^ ((r ^ (r >> 3)) & 7) (realized by choosing each lane's source
//    address, since a DMA instruction writes 1 KB contiguously), keeping the
//    16-row operand reads free of bank conflicts for 32 and 64 banks.
//  * persistent grid (one workgroup per CU): each workgroup strides over the
//    output tiles; a tile's expert is found by binary search over the
//    segment offsets (segments are multiples of 128 rows, so a tile never
//    straddles two experts).
#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

namespace {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int kWavesN = 4;                       // 2 x 4 waves, each 64 x 64
constexpr int kWaves = 2 * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveCols = BN / kWavesN;          // 64
constexpr int kNFrag = kWaveCols / 16;           // 4 MFMA column subtiles per wave
constexpr int kStages = 3;
constexpr int kABytes = BM * BK;                 // 16 KB
constexpr int kBBytes = BN * BK;                 // 32 KB
constexpr int kSBytes = BM * 4;                  // 512 B of activation scales
constexpr int kStageBytes = kABytes + kBBytes + kSBytes;
constexpr int kADma = kABytes / 1024 / kWaves;   // 16-byte-per-lane DMA instructions per wave
constexpr int kBDma = kBBytes / 1024 / kWaves;
constexpr int kSRows = BM / kWaves;              // activation scales per wave (dword DMA lanes)
constexpr int kDmaPerStage = kADma + kBDma + 1;

__device__ inline int swz(int row) { return (row ^ (row >> 3)) & 7; }

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

template <int N>
__device__ inline void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ inline void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

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

__global__ void __launch_bounds__(kThreads, 1)
gemm_fp8_contig_kernel(int G, int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
                       const float* __restrict__ SA, const uint8_t* __restrict__ B,
                       const float* __restrict__ SB, const int32_t* __restrict__ offsets,
                       uint16_t* __restrict__ D, int64_t ldd) {
  __shared__ __align__(16) uint8_t smem[kStages * kStageBytes];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;      // 2 waves along M, kWavesN along N
  const int l16 = lane & 15, q = lane >> 4;

  const int64_t m_end = offsets ? (int64_t)offsets[G] : M;
  const int64_t m_tiles = (m_end + BM - 1) / BM;
  const int64_t n_tiles = (N + BN - 1) / BN;     // N % 128 == 0: a last tile may be half wide
  const int64_t num_tiles = m_tiles * n_tiles;
  const int nkb = (int)(K / BK);
  const int64_t nblk = N / 128;

  // DMA lane roles: lane l fills 16-byte LDS chunk (l % 8) of row (l / 8) of an 8-row group;
  // it reads source chunk (l % 8) ^ swz(row), where swz(row) = (l / 8) ^ (row-group index & 7).
  const int lrow = lane >> 3;
  const int lchunk = (lane & 7) ^ lrow;

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
    const int64_t rows_here = (m_end - m0) < BM ? (m_end - m0) : BM;   // >= 1
    const int64_t cols_here = (N - n0) < BN ? (N - n0) : BN;           // 128 or 256
    const uint8_t* Atile = A + m0 * K;
    const uint8_t* Btile = B + ((int64_t)g * N + n0) * K;
    const int64_t nb_w = (n0 + wn * kWaveCols) / 128;
    const int64_t nb = nb_w < nblk ? nb_w : (nblk - 1);
    const float* SBw = SB + ((int64_t)g * nblk + nb) * nkb;

    // per-lane byte offsets (within the tile) of this wave's DMA rows; rows past the
    // end of A are redirected to the last valid row (their outputs are never stored)
    uint32_t offA[kADma], offB[kBDma];
#pragma unroll
    for (int i = 0; i < kADma; ++i) {
      const int grp8 = wave * kADma + i;             // 8-row group of the A tile
      int row = grp8 * 8 + lrow;
      const int c = lchunk ^ (grp8 & 7);
      if (row >= rows_here) row = (int)rows_here - 1;
      offA[i] = (uint32_t)(row * K + c * 16);
    }
#pragma unroll
    for (int i = 0; i < kBDma; ++i) {
      const int grp8 = wave * kBDma + i;
      int row = grp8 * 8 + lrow;
      const int c = lchunk ^ (grp8 & 7);
      if (row >= cols_here) row = (int)cols_here - 1;   // half-wide last tile: stay inside B
      offB[i] = (uint32_t)(row * K + c * 16);
    }
    int srow = wave * kSRows + (lane % kSRows);
    if (srow >= rows_here) srow = (int)rows_here - 1;
    const uint32_t offS = (uint32_t)(srow * 4);

    auto issue = [&](int kb, int stage) {
      const uint32_t st = lds_base + stage * kStageBytes;
      const uint8_t* a_src = Atile + (int64_t)kb * BK;
      const uint8_t* b_src = Btile + (int64_t)kb * BK;
#pragma unroll
      for (int i = 0; i < kADma; ++i) dma16(a_src, offA[i], st + (wave * kADma + i) * 1024);
#pragma unroll
      for (int i = 0; i < kBDma; ++i) dma16(b_src, offB[i], st + kABytes + (wave * kBDma + i) * 1024);
      // kSRows scales per wave: the first kSRows lanes only (still one DMA instruction per wave)
      const float* s_src = SA + (int64_t)kb * M + m0;
      if (lane < kSRows) dma4(s_src, offS, st + kABytes + kBBytes + wave * kSRows * 4);
    };

    v4f acc[4][kNFrag];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kNFrag; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    block_barrier();          // every wave is done with the previous tile's LDS
    issue(0, 0);
    if (nkb > 1) issue(1, 1);

    for (int kb = 0; kb < nkb; ++kb) {
      if (kb + 1 < nkb) wait_vmcnt<kDmaPerStage>();   // stage kb landed (kb+1 may still fly)
      else wait_vmcnt<0>();
      block_barrier();                                 // ... for all waves; stage (kb+2)%3 is free
      if (kb + 2 < nkb) issue(kb + 2, (kb + 2) % kStages);

      const int stage = kb % kStages;
      const uint8_t* At = smem + stage * kStageBytes;
      const uint8_t* Bt = At + kABytes;
      const float* St = reinterpret_cast<const float*>(Bt + kBBytes);
      const float sb = SBw[kb];

      v8i af[4];
      float sab[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i] = read_frag(At, wm * 64 + 16 * i + l16, q);
        sab[i] = St[wm * 64 + 16 * i + l16] * sb;
      }
#pragma unroll
      for (int h = 0; h < kNFrag / 4; ++h) {
        v8i bf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bf[j] = read_frag(Bt, wn * kWaveCols + 16 * (4 * h + j) + l16, q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                bf[j], af[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
            v4f& c = acc[i][4 * h + j];
            c[0] = fmaf(p[0], sab[i], c[0]);
            c[1] = fmaf(p[1], sab[i], c[1]);
            c[2] = fmaf(p[2], sab[i], c[2]);
            c[3] = fmaf(p[3], sab[i], c[3]);
          }
        }
      }
    }

    // epilogue: lane holds columns n0 + wn*64 + 16j + 4q + (0..3) of row m0 + wm*64 + 16i + l16
    if (wn * kWaveCols >= cols_here) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + wm * 64 + 16 * i + l16;
      if (row >= m_end) continue;
      uint16_t* drow = D + row * ldd + n0 + wn * kWaveCols + 4 * q;
#pragma unroll
      for (int j = 0; j < kNFrag; ++j) {
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
  if (N % 128 != 0 || K % BK != 0) return hipErrorInvalidValue;
  const int64_t tiles_upper = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int64_t grid = (int64_t)num_cus;
  if (grid > tiles_upper) grid = tiles_upper;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(gemm_fp8_contig_kernel, dim3((unsigned)grid), dim3(kThreads), 0, st, G, M, N, K, a, sa, b,
                     sb, offsets, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
