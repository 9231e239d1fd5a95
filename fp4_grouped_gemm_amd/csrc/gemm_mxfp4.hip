// MXFP4 W4A4 GEMM with the low-rank residual and per-column bias:
//   Y = (Q(X) · Q(W)ᵀ) ⊙ scale + L(X) + b,     L(X) = (X · L_down) · L_up
// ([W4A4] "最新GPU架构上W4A4算子的Warp专用化内核实践" §1, operator equation), with Q the
// MX form: E2M1 codes and one E8M0 power-of-two scale per 32 elements along K, on both
// operands.  ⊙ scale then applies 2^(eX-127) · 2^(eW-127) to every 32-element partial
// sum, which is exactly what gfx950's block-scaled matrix instruction does in hardware:
// v_mfma_scale_f32_16x16x128_f8f6f4 with both formats FP4 takes each lane's E8M0 byte
// for the 32 K elements that lane holds.  So, unlike the per-16 fp32-scale path, nothing
// is dequantized and nothing is promoted on the vector ALU: the K loop is FP4 MFMAs
// accumulating in place, at the FP4 rate (measured on MI355X from registers only:
// 8.1-8.7 PFLOP/s, twice the FP8 rate).
//
// Tile 256 x 192 per 512-thread workgroup (4096 x 3072 is exactly 256 tiles, one per
// CU), eight waves (two per SIMD) of 128 x 48 outputs: 8 x 3 MFMA tiles, 96 fp32
// accumulators per lane.  A K stage is one 128-wide K block: 256 A rows and 192 B rows
// of 64 code bytes (E2M1 pairs) plus one scale dword (four E8M0 bytes) per row,
// 29.75 KB (padded to 30 KB); four stages in a ring (120 KB), filled by global_load_lds
// (gfx950's direct global->LDS path) three stages ahead.  Every wave issues exactly five
// DMA instructions per stage (A codes 2, then B codes 2 and B scales 1 for waves 0-3, B
// codes 1 and A scales 2 for waves 4-7), so its hand-counted vmcnt waits are the same
// constants.  A
// 64-byte row's four 16-byte chunks are XOR-swizzled with key(row) = 2·bit2(row) ^
// 3·bit3(row): gfx950 serves a ds_read_b128 in four cycles of 16 lanes each, lanes
// {0-3, 12-15, 20-23, 24-27} (+32) in one and {4-11, 16-19, 28-31} (+32) in another
// (measured with SQ_LDS_BANK_CONFLICT), so a cycle mixes rows of two lane groups q; with
// this key those 16 lanes hit 16 distinct 16-byte slots of the 64 banks (the former key
// (row >> 2) & 3 was conflict-free for 16 consecutive lanes only and doubled every
// fragment read).
//
// Fragments (16x16x128, FP4): lane (l16, q) holds bytes [16q, 16q+16) of row l16 of the
// 16-row tile (K elements [32q, 32q+32) of the block) and byte q of that row's scale
// dword.  The weight tile is the first operand, so a lane's four results are four
// consecutive columns of one row (8-byte bf16 stores).
//
// The low-rank branch: T = X·L_down ([M][32] bf16, by w4a4_lowrank_kernel in
// gemm_w4a4.hip) before the GEMM, and one bf16 MFMA step T·L_up (K = 32)
// into the accumulators of each output tile before the bias is added.
#include <type_traits>

#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace mx {
constexpr int BM = 256, BN = 192, BK = 128;
constexpr int kRowBytes = BK / 2;                 // 64 code bytes per row and K block
constexpr int kABytes = BM * kRowBytes;           // 16 KB
constexpr int kBBytes = BN * kRowBytes;           // 12 KB
constexpr int kSAOff = kABytes + kBBytes;         // A scales: one dword per row
constexpr int kSBOff = kSAOff + BM * 4;           // B scales
constexpr int kStageBytes = (kSBOff + BN * 4 + 1023) / 1024 * 1024;   // 30464 used, padded to 30 KB
constexpr int kStages = 4;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kWM = 128, kWN = 48;                // a wave's outputs
constexpr int kMI = kWM / 16, kNJ = kWN / 16;     // 8 x 3 MFMA tiles
constexpr int kDmaPerWave = 5;                    // DMA instructions per wave per stage
constexpr int kGM = 4;                            // tile rows per raster group
static_assert(kStages * kStageBytes <= 160 * 1024, "LDS budget");
static_assert(kStageBytes % 16 == 0, "stage alignment");
__device__ inline int key(int row) { return (((row >> 2) & 1) * 2) ^ (((row >> 3) & 1) * 3); }

}  // namespace mx

__global__ void __launch_bounds__(mx::kThreads, 1)
gemm_mxfp4_kernel(int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB, const uint16_t* __restrict__ T,
                  const uint16_t* __restrict__ Lu, int rank, const uint16_t* __restrict__ bias,
                  uint16_t* __restrict__ D, int64_t ldd) {
  using namespace mx;
  __shared__ __align__(16) uint8_t smem[kStages * kStageBytes];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;        // waves w and w + 4 (one SIMD) take the two row halves
  const int l16 = lane & 15, q = lane >> 4;

  // Tile order: consecutive tile indices go to one XCD (workgroup b runs on XCD b % 8),
  // rastered in groups of kGM tile rows, so an XCD's tiles share A and B blocks in its L2.
  const int64_t nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN, tiles = nM * nN;
  const int64_t per_xcd = (tiles + 7) / 8;
  const int64_t t = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (t >= tiles) return;
  const int64_t group = t / (kGM * nN), first_m = group * kGM;
  const int64_t gm = (nM - first_m) < kGM ? (nM - first_m) : kGM;
  const int64_t idx = t - group * kGM * nN;
  const int64_t m0 = (first_m + idx % gm) * BM, n0 = (idx / gm) * BN;
  const int rows = (int)((M - m0) < BM ? (M - m0) : BM), cols = (int)((N - n0) < BN ? (N - n0) : BN);
  const int nkb = (int)(K / BK);
  const uint32_t kbytes = (uint32_t)(K / 2), kscales = (uint32_t)(K / 32);

  // DMA roles (wave-uniform) and this lane's source offsets.  A code segment s (16 rows
  // of 64 bytes = 1 KB): lane l fills chunk l % 4 of row 16 s + l / 4 and reads source
  // chunk (l % 4) ^ key(row).  Rows past the tile's end read its last valid row (never
  // stored).
  const uint8_t* Abase = A + m0 * (int64_t)kbytes;
  const uint8_t* Bbase = B + n0 * (int64_t)kbytes;
  const uint8_t* SAbase = SA + m0 * (int64_t)kscales;
  const uint8_t* SBbase = SB + n0 * (int64_t)kscales;
  const int lrow = lane >> 2, lpos = lane & 3;
  auto code_off = [&](int seg, int lim) -> uint32_t {
    const int row = seg * 16 + lrow;
    const int src = row < lim ? row : lim - 1;
    return (uint32_t)src * kbytes + (uint32_t)((lpos ^ key(row)) * 16);
  };
  const int a_seg0 = 2 * wave;                                  // A code segments 2w, 2w + 1
  const int b_seg0 = wave < 4 ? 2 * wave : 8 + (wave - 4);      // B code segments
  const uint32_t oa0 = code_off(a_seg0, rows), oa1 = code_off(a_seg0 + 1, rows);
  const uint32_t ob0 = code_off(b_seg0, cols), ob1 = code_off(wave < 4 ? b_seg0 + 1 : b_seg0, cols);
  // scale rows: waves 0-3 fetch B rows [48 w, 48 w + 48) (lanes < 48); waves 4-7 fetch A rows
  // [64 (w - 4), 64 (w - 4) + 64) as two instructions of 32 lanes
  int srow0, srow1 = 0;
  if (wave < 4) {
    srow0 = 48 * wave + lane;
    if (srow0 >= cols) srow0 = cols - 1;
  } else {
    srow0 = 64 * (wave - 4) + (lane & 31);
    srow1 = srow0 + 32;
    if (srow0 >= rows) srow0 = rows - 1;
    if (srow1 >= rows) srow1 = rows - 1;
  }
  const uint32_t os0 = (uint32_t)srow0 * kscales, os1 = (uint32_t)srow1 * kscales;

  auto issue = [&](int kb, int stage) {
    const uint32_t sbase = lds_base + stage * kStageBytes;
    const uint8_t* asrc = Abase + (int64_t)kb * kRowBytes;
    const uint8_t* bsrc = Bbase + (int64_t)kb * kRowBytes;
    dma16(asrc, oa0, sbase + a_seg0 * 1024);
    dma16(asrc, oa1, sbase + (a_seg0 + 1) * 1024);
    if (wave < 4) {
      dma16(bsrc, ob0, sbase + kABytes + b_seg0 * 1024);
      dma16(bsrc, ob1, sbase + kABytes + (b_seg0 + 1) * 1024);
      if (lane < 48) dma4(SBbase + (int64_t)kb * 4, os0, sbase + kSBOff + 48 * wave * 4);
    } else {
      dma16(bsrc, ob0, sbase + kABytes + b_seg0 * 1024);
      const uint32_t sa = sbase + kSAOff + 64 * (wave - 4) * 4;
      if (lane < 32) dma4(SAbase + (int64_t)kb * 4, os0, sa);
      if (lane < 32) dma4(SAbase + (int64_t)kb * 4, os1, sa + 128);
    }
  };

  v4f acc[kMI][kNJ];
#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // this lane's fragment addresses within a stage: row 16 i (A) / 16 j (B) further is
  // 1024 bytes further, with the same swizzle key (key depends on l16 only)
  const int arow = wm * kWM + l16, brow = wn * kWN + l16;
  const uint32_t ra = (uint32_t)(arow * kRowBytes + ((q ^ key(arow)) << 4));
  const uint32_t rb = (uint32_t)(kABytes + brow * kRowBytes + ((q ^ key(brow)) << 4));
  const uint32_t rsa = (uint32_t)(kSAOff + arow * 4), rsb = (uint32_t)(kSBOff + brow * 4);
  const bool live = (wm * kWM < rows) && (wn * kWN < cols);

  auto step = [&](int stage) {
    const uint8_t* s = smem + stage * kStageBytes;
    uint4 af[kMI], bf[kNJ];
    uint32_t sa[kMI], sb[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      bf[j] = *reinterpret_cast<const uint4*>(s + rb + j * 1024);
      sb[j] = *reinterpret_cast<const uint32_t*>(s + rsb + j * 64);
    }
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      af[i] = *reinterpret_cast<const uint4*>(s + ra + i * 1024);
      sa[i] = *reinterpret_cast<const uint32_t*>(s + rsa + i * 64);
    }
    int eb[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) eb[j] = (int)__builtin_amdgcn_ubfe(sb[j], 8 * q, 8);
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      const int ea = (int)__builtin_amdgcn_ubfe(sa[i], 8 * q, 8);
      const v8i a8 = v8i{(int)af[i].x, (int)af[i].y, (int)af[i].z, (int)af[i].w, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < kNJ; ++j) {
        const v8i b8 = v8i{(int)bf[j].x, (int)bf[j].y, (int)bf[j].z, (int)bf[j].w, 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b8, a8, acc[i][j], 4, 4, 0, eb[j], 0, ea);
      }
    }
  };

  // top of step kb: this wave's DMA of stage kb landed (stages kb + 1, kb + 2 may fly);
  // the barrier makes that true for every wave and proves every wave has finished
  // reading stage kb - 1 (its fragments were consumed by the MFMAs of step kb - 1), so
  // that stage's buffer takes stage kb + 3.
  if (nkb > 0) issue(0, 0);
  if (nkb > 1) issue(1, 1);
  if (nkb > 2) issue(2, 2);
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 2 < nkb) wait_vmcnt<2 * kDmaPerWave>();
    else if (kb + 1 < nkb) wait_vmcnt<kDmaPerWave>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (kb + 3 < nkb) issue(kb + 3, (kb + 3) & 3);
    if (live) step(kb & 3);
  }
  if (!live) return;

  // low-rank step: acc += T[m][0:32] · L_up[0:32][n]  (one bf16 MFMA K step of 32)
  if (rank == 32) {
    v8bf lf[kNJ];
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      int64_t n = n0 + wn * kWN + 16 * j + l16;
      if (n >= N) n = N - 1;
      uint16_t u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = Lu[(int64_t)(8 * q + e) * N + n];
      lf[j] = __builtin_bit_cast(v8bf, u);
    }
#pragma unroll
    for (int i = 0; i < kMI; ++i) {
      int64_t m = m0 + wm * kWM + 16 * i + l16;
      if (m >= M) m = M - 1;
      const v8bf tf = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(T + m * 32 + 8 * q));
#pragma unroll
      for (int j = 0; j < kNJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lf[j], tf, acc[i][j], 0, 0, 0);
    }
  }

  // lane (l16, q) holds columns n0 + 48 wn + 16 j + 4 q + (0..3) of row m0 + 128 wm + 16 i + l16
  float bv[kNJ][4];
#pragma unroll
  for (int j = 0; j < kNJ; ++j) {
    const int64_t n = n0 + wn * kWN + 16 * j + 4 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[j][e] = (bias && n < N) ? bf16_to_f32(bias[n + e]) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kMI; ++i) {
    const int64_t row = m0 + wm * kWM + 16 * i + l16;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      const int64_t n = n0 + wn * kWN + 16 * j + 4 * q;
      if (n >= N) continue;                         // N % 16 == 0: a lane's 4 columns are all in or all out
      const uint32_t lo = bf16x2_rne(acc[i][j][0] + bv[j][0], acc[i][j][1] + bv[j][1]);
      const uint32_t hi = bf16x2_rne(acc[i][j][2] + bv[j][2], acc[i][j][3] + bv[j][3]);
      *reinterpret_cast<uint2*>(D + row * ldd + n) = make_uint2(lo, hi);
    }
  }
}

size_t mxfp4_workspace_bytes(int64_t M, int32_t rank) { return rank > 0 ? (size_t)M * 32 * 2 : 0; }

const KernelInfo kInfoMxfp4Gemm = {"gemm_mxfp4_kernel", "fgg_scaled_gemm (MXFP4: E2M1 + E8M0/32 on both operands)",
                                   mx::BM, mx::BN, mx::BK, mx::kThreads, mx::kStages, mx::kStageBytes, 0,
                                   mx::kStages * mx::kStageBytes, (const void*)gemm_mxfp4_kernel};

hipError_t launch_mxfp4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                        const uint8_t* sb, const uint16_t* x_bf16, const uint16_t* l_down, const uint16_t* l_up,
                        int32_t rank, const uint16_t* bias, uint16_t* d, int64_t ldd, void* ws, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (N % 16 != 0 || K % 128 != 0 || K == 0) return hipErrorInvalidValue;
  uint16_t* T = rank > 0 ? reinterpret_cast<uint16_t*>(ws) : nullptr;
  if (rank > 0) {
    const hipError_t e = launch_lowrank_t(M, K, x_bf16, l_down, T, st);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = ((M + mx::BM - 1) / mx::BM) * ((N + mx::BN - 1) / mx::BN);
  const int64_t grid = (tiles + 7) / 8 * 8;          // a multiple of the XCD count (tile order above)
  trace_launch(kInfoMxfp4Gemm, dim3((unsigned)grid), "M=%lld N=%lld K=%lld rank=%d%s", (long long)M, (long long)N,
               (long long)K, (int)rank, bias ? " bias" : "");
  hipLaunchKernelGGL(gemm_mxfp4_kernel, dim3((unsigned)grid), dim3(mx::kThreads), 0, st, M, N, K, a, sa, b, sb, T,
                     l_up, (int)rank, bias, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
