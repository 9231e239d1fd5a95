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
// The low-rank branch is T = X·L_down on bf16 MFMA (fp32 accumulate, stored bf16
// in the workspace), computed by its own blocks of the operand-preparation launch,
// and one extra bf16 MFMA step T·L_up per output tile, before the bias is added in
// the epilogue.
//
// GEMM tile: 256 x 192 per 1024-thread workgroup, four waves per SIMD, each wave 64 x 48
// outputs (48 fp32 accumulators); two LDS buffers of 64-wide K stages filled by
// global_load_lds_dwordx4 one stage ahead (details at the kernel).  Measured on MI355X,
// v_mfma_f32_16x16x32_f16 issues at 2.3-2.4 PFLOP/s from registers with constant
// operands and at 1.6-1.7 PFLOP/s with random ones (the clock drops under the switching
// load); this GEMM reaches about 1.0 PFLOP/s: with one 256 x 192 tile per CU (4096 x
// 3072) the pipeline fill and the epilogue are not hidden.  The
// MXFP4 form (gemm_mxfp4.hip) runs the scaled FP4 MFMA on the codes directly instead.
#include <algorithm>
#include <type_traits>

#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {
__device__ inline float e2m1_f32(uint32_t nib, float s) {
  const uint32_t mag = nib & 7u;
  float f = __uint_as_float((mag + 252u) << 22);        // exact for magnitude codes >= 2
  f = (mag < 2u) ? 0.5f * (float)mag : f;              // 0 and 0.5
  f = (nib & 8u) ? -f : f;
  return f * s;
}

}  // namespace

// The low-rank intermediate T[m][r] = Σ_k X[m][k] · L_down[k][r] (rank 32) for the 16
// rows of block blk, fp32 accumulate, stored bf16, by the block's W waves.  K is cut
// into 32-wide chunks, chunk c summed by wave c % W with v_mfma_f32_16x16x32_bf16
// (first operand: 16 ranks of L_down, second: the 16 X rows; lane (l, q) holds K
// elements [8q, 8q+8) of row l of each), two rank tiles per wave.  A wave loads the X
// fragments and L_down slices of kBatch chunks before using any, so that their reads
// are in flight together (the branch is bound by the latency of these reads, not by
// their bytes).  L_down is [K][32] (ranks contiguous): each 32-row slice is written
// transposed into the wave's own LDS area ldt[wave] ([32 ranks][32 k]), from which
// the rank-major fragments are read (a wave's LDS operations take effect in program
// order).  The W partial sums are added in wave order through part.
constexpr int kBatch = 4;

template <int W>
__device__ inline void lowrank_rows(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Ld,
                                    uint16_t* __restrict__ T, int64_t M, int64_t K, int64_t blk,
                                    uint16_t (*ldt)[32 * 32], v4f (*part)[2][64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t m0 = blk * 16;
  int64_t mrow = m0 + l16;
  if (mrow >= M) mrow = M - 1;               // rows past the end read a valid row; never stored
  const int nch = (int)(K / 32);             // chunks; wave w takes w, w + W, ...
  const uint16_t* xr = X + mrow * K + 8 * q;
  uint16_t* tl = ldt[wave];
  const int kk = lane >> 1, rb = 16 * (lane & 1);   // the L_down elements this lane moves
  const bool ld_vec = (reinterpret_cast<uintptr_t>(Ld) & 15u) == 0;
  v4f acc0 = v4f{0.f, 0.f, 0.f, 0.f}, acc1 = v4f{0.f, 0.f, 0.f, 0.f};
  for (int c0 = wave; c0 < nch; c0 += W * kBatch) {
    uint4 xa[kBatch], r0[kBatch], r1[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * W;
      if (c < nch) {
        xa[b] = *reinterpret_cast<const uint4*>(xr + (int64_t)c * 32);
        if (ld_vec) {
          const uint16_t* src = Ld + ((int64_t)c * 32 + kk) * 32 + rb;   // row 32c + kk, ranks rb .. rb + 15
          r0[b] = *reinterpret_cast<const uint4*>(src);
          r1[b] = *reinterpret_cast<const uint4*>(src + 8);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * W;
      if (c >= nch) break;
      if (ld_vec) {
        const uint32_t w[8] = {r0[b].x, r0[b].y, r0[b].z, r0[b].w, r1[b].x, r1[b].y, r1[b].z, r1[b].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          tl[(rb + 2 * e) * 32 + kk] = (uint16_t)(w[e] & 0xFFFFu);
          tl[(rb + 2 * e + 1) * 32 + kk] = (uint16_t)(w[e] >> 16);
        }
      } else {                                        // L_down only 2-byte aligned
        const uint16_t* src = Ld + ((int64_t)c * 32 + kk) * 32 + rb;
#pragma unroll
        for (int e = 0; e < 16; ++e) tl[(rb + e) * 32 + kk] = src[e];
      }
      const uint4 la = *reinterpret_cast<const uint4*>(tl + l16 * 32 + 8 * q);
      const uint4 lb = *reinterpret_cast<const uint4*>(tl + (16 + l16) * 32 + 8 * q);
      const v8bf xv = __builtin_bit_cast(v8bf, xa[b]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, la), xv, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, lb), xv, acc1, 0, 0, 0);
    }
  }
  part[wave][0][lane] = acc0;
  part[wave][1][lane] = acc1;
  __syncthreads();
  if (wave != 0) return;
  // lane (l16, q) holds ranks 4q..4q+3 (tile 0) and 16+4q.. (tile 1) of row m0 + l16
  v4f s0 = part[0][0][lane], s1 = part[0][1][lane];
#pragma unroll
  for (int w = 1; w < W; ++w) {
    const v4f a = part[w][0][lane], b = part[w][1][lane];
    s0[0] += a[0]; s0[1] += a[1]; s0[2] += a[2]; s0[3] += a[3];
    s1[0] += b[0]; s1[1] += b[1]; s1[2] += b[2]; s1[3] += b[3];
  }
  const int64_t m = m0 + l16;
  if (m >= M) return;
  uint16_t* t = T + m * 32 + 4 * q;
  *reinterpret_cast<uint2*>(t) = make_uint2(bf16x2_rne(s0[0], s0[1]),
                                            bf16x2_rne(s0[2], s0[3]));
  *reinterpret_cast<uint2*>(t + 16) = make_uint2(bf16x2_rne(s1[0], s1[1]),
                                                 bf16x2_rne(s1[2], s1[3]));
}

// The GEMM's operand preparation and the low-rank branch in one launch, by block
// ranges, so that the two run side by side:
//  * blocks [0, M/16) (with the low-rank branch): lowrank_rows with four waves;
//  * the following blocks: packed E2M1 rows with fp32 scales per 16 -> fp16 (x·s
//    rounded once), for A ([M][K/2] -> [M][K]) and B, 8 elements per item (4 code
//    bytes in, 16 bytes out), kItems items per thread at a stride of 256 so that each
//    store instruction writes consecutive 16-byte pieces and every load of a thread is
//    in flight before its first conversion.
// Without the dequantization (the MXFP4 form), the low-rank branch runs alone in
// w4a4_lowrank_kernel, with sixteen waves per 16 rows: more reads in flight per row.
constexpr int kItems = 4;
constexpr int kLrWaves = 4;
constexpr int kLrWavesAlone = 16;

__device__ inline void dequant_items(const uint8_t* __restrict__ q, const float* __restrict__ s, int64_t base,
                                     int64_t n, uint16_t* __restrict__ out) {
  uint32_t w[kItems];
  float sc[kItems];
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t i = base + 256 * j;
    if (i < n) {
      w[j] = *reinterpret_cast<const uint32_t*>(q + i * 4);
      sc[j] = s[i >> 1];                          // elements 8i..8i+7 lie in 16-element group i/2
    }
  }
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int64_t i = base + 256 * j;
    if (i >= n) break;
    uint32_t h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (w[j] >> (8 * b)) & 0xFFu;
      const _Float16 lo = (_Float16)e2m1_f32(byte & 0xFu, sc[j]);
      const _Float16 hi = (_Float16)e2m1_f32(byte >> 4, sc[j]);
      h[b] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<uint4*>(out + i * 8) = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

__global__ void __launch_bounds__(256) w4a4_prep_kernel(const uint8_t* __restrict__ qa, const float* __restrict__ sa,
                                                        int64_t na, uint16_t* __restrict__ ah,
                                                        const uint8_t* __restrict__ qb, const float* __restrict__ sb,
                                                        int64_t nb, uint16_t* __restrict__ bh,
                                                        const uint16_t* __restrict__ X, const uint16_t* __restrict__ Ld,
                                                        uint16_t* __restrict__ T, int64_t M, int64_t K,
                                                        int64_t lr_blocks) {
  __shared__ __align__(16) uint16_t ldt[kLrWaves][32 * 32];
  __shared__ v4f part[kLrWaves][2][64];
  constexpr int64_t kPer = 256 * kItems;
  const int64_t blk = blockIdx.x;
  if (blk >= lr_blocks) {
    const int64_t ba = (na + kPer - 1) / kPer;
    const int64_t pb = blk - lr_blocks;
    if (pb < ba) dequant_items(qa, sa, pb * kPer + threadIdx.x, na, ah);
    else dequant_items(qb, sb, (pb - ba) * kPer + threadIdx.x, nb, bh);
    return;
  }
  lowrank_rows<kLrWaves>(X, Ld, T, M, K, blk, ldt, part);
}

__global__ void __launch_bounds__(64 * kLrWavesAlone) w4a4_lowrank_kernel(const uint16_t* __restrict__ X,
                                                                          const uint16_t* __restrict__ Ld,
                                                                          uint16_t* __restrict__ T, int64_t M,
                                                                          int64_t K) {
  __shared__ __align__(16) uint16_t ldt[kLrWavesAlone][32 * 32];
  __shared__ v4f part[kLrWavesAlone][2][64];
  lowrank_rows<kLrWavesAlone>(X, Ld, T, M, K, blockIdx.x, ldt, part);
}

// The fp16 GEMM D = A_h · B_hᵀ (+ T · L_up) (+ bias), bf16 out.  Workgroup tile 256 x 192,
// sixteen waves (four per SIMD) of 64 x 48 outputs: 4 x 3 MFMA subtiles, 48 fp32
// accumulators per lane, at most 128 VGPRs per wave.  Measured alternatives on the same
// tile: one wave per SIMD (128 x 96 each, accumulators in the accumulation registers,
// 299 bytes of LDS reads per MFMA) 16% slower for the whole call, two per SIMD (128 x 48)
// 5% slower: a SIMD's other waves issue MFMAs while one waits at the barrier or issues
// its DMA.  The 4096 x 3072 shape is exactly 256 tiles, one per CU.
// K stages of 64 (two MFMA steps): 256 A rows + 192 B rows of 128 bytes = 56 KB, two
// buffers, the DMA of stage ks + 1 (waves 0-7, 7 instructions each) issued right after the
// barrier of step ks; a step reads both halves' fragments at its top and runs 24 MFMAs
// (the SIMD's other waves cover the read latency).  Measured against a 4-buffer ring of
// 32-wide stages two ahead with the next stage's fragments read during the current
// MFMAs: 4% faster for the whole call (half the barriers).  A 128-byte row's eight
// 16-byte chunks are XOR-swizzled with key(row) = bit1(row) ^ 4·bit2(row) ^ 6·bit3(row):
// gfx950 serves a ds_read_b128 in four cycles of 16 lanes, lanes {0-3, 12-15, 20-23,
// 24-27} (+32) in one and {4-11, 16-19, 28-31} (+32) in another (measured), so a cycle
// holds rows of lane groups q and q + 1 reading chunks 4h + q and 4h + q + 1; this key
// puts those 16 lanes on 16 distinct 16-byte slots of the 64 banks (the former key
// (row & 7) ^ ((row >> 3) & 1) left two lanes on each slot: 8 cycles per read instead
// of 4).  Rows past M or N read the last valid row (never stored).
namespace w4 {
constexpr int BM = 256, BN = 192, BK = 64;
constexpr int kRowBytes = BK * 2;                 // 128
constexpr int kABytes = BM * kRowBytes;           // 32 KB
constexpr int kStageBytes = (BM + BN) * kRowBytes;  // 56 KB
constexpr int kStages = 2;
constexpr int kWaves = 16;                        // four per SIMD: 4 row x 4 column waves
constexpr int kDmaWaves = 8;                      // waves 0-7 issue the stage DMA
constexpr int kDma = kStageBytes / 1024 / kDmaWaves; // 7
constexpr int kWC = 48, kNJ = 3;                  // a wave's columns and column subtiles (64 rows)
constexpr int kAGroups = kABytes / 1024;          // 32 (8 rows per KB)
constexpr int kGM = 4;                            // tile rows per raster group
static_assert(kStages * kStageBytes <= 160 * 1024, "LDS budget");
__device__ inline int key(int row) { return ((row >> 1) & 1) ^ (((row >> 2) & 1) * 4) ^ (((row >> 3) & 1) * 6); }
}  // namespace w4

__global__ void __launch_bounds__(1024, 1)
w4a4_gemm_kernel(int64_t M, int64_t N, int64_t K, const uint16_t* __restrict__ Ah, const uint16_t* __restrict__ Bh,
                 const uint16_t* __restrict__ T, const uint16_t* __restrict__ Lu, int rank,
                 const uint16_t* __restrict__ bias, uint16_t* __restrict__ D, int64_t ldd) {
  using namespace w4;
  __shared__ __align__(16) uint8_t smem[kStages * kStageBytes];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;      // 64 rows, 48 columns each
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
  const bool live = (wm * 64 < rows) && (wn * kWC < cols);
  const int nks = (int)(K / BK);

  // DMA roles: a stage is 56 segments of 1 KB (8 rows of 128 bytes), segments 0-31 the A
  // rows, 32-55 the B rows; wave w < 8 issues segments 7w .. 7w+6 (the other waves none,
  // so their vmcnt waits return at once).  Lane l fills chunk l % 8 of row l / 8 of its
  // segment and reads source chunk (l % 8) ^ key(row).
  const uint8_t* Abase = reinterpret_cast<const uint8_t*>(Ah + m0 * K);
  const uint8_t* Bbase = reinterpret_cast<const uint8_t*>(Bh + n0 * K);
  uint32_t voff[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int seg = wave * kDma + i;
    const int row = seg * 8 + (lane >> 3);           // row of the stage ([A rows][B rows])
    int src = seg < kAGroups ? row : row - BM;
    const int lim = seg < kAGroups ? rows : cols;
    if (src >= lim) src = lim - 1;
    voff[i] = (uint32_t)src * (uint32_t)(K * 2) + (uint32_t)((((lane & 7) ^ key(row))) * 16);
  }
  auto issue = [&](int ks, int stage) {
    if (wave >= kDmaWaves) return;
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int seg = wave * kDma + i;               // wave-uniform
      const uint8_t* src = (seg < kAGroups ? Abase : Bbase) + (int64_t)ks * (BK * 2);
      dma16(src, voff[i], lds_base + stage * kStageBytes + seg * 1024);
    }
  };

  v4f acc[4][kNJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kNJ; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // fragments: lane (l16, q) takes 8 fp16 (K [32h + 8q, 32h + 8q + 8) of half h of the
  // stage) of rows 16 i + l16 of the wave's A rows and of its B rows; rows 16 apart share
  // a swizzle key
  const int arow = wm * 64 + l16, brow = BM + wn * kWC + l16;
  struct Frags {
    v8h a[4], b[kNJ];
  };
  auto read_frags = [&](int slot, int h, Frags& f) {
    const uint8_t* base = smem + slot * kStageBytes;
    const int ao = arow * kRowBytes + (((4 * h + q) ^ key(arow)) << 4);
    const int bo = brow * kRowBytes + (((4 * h + q) ^ key(brow)) << 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const v8h*>(base + ao + 16 * i * kRowBytes);
#pragma unroll
    for (int j = 0; j < kNJ; ++j) f.b[j] = *reinterpret_cast<const v8h*>(base + bo + 16 * j * kRowBytes);
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };
  // top of step ks: this wave's DMA of stage ks landed and its reads of the other buffer
  // (step ks - 1) done; the barrier makes both true for every wave, so stage ks is
  // readable and the other buffer takes stage ks + 1.  Both halves' fragments are read
  // at the top (the other waves of the SIMD cover the latency).
  if (nks > 0) issue(0, 0);
  for (int ks = 0; ks < nks; ++ks) {
    wait_vmcnt<0>();
    __syncthreads();
    if (ks + 1 < nks) issue(ks + 1, (ks + 1) & 1);
    if (live) {
      Frags f0, f1;
      read_frags(ks & 1, 0, f0);
      read_frags(ks & 1, 1, f1);
      mma(f0);
      mma(f1);
    }
  }
  if (!live) return;

  // low-rank step: acc += T[m][0:32] · L_up[0:32][n]  (one bf16 MFMA K step of 32)
  if (rank == 32) {
    v8bf tf[4], lf[kNJ];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t m = m0 + wm * 64 + 16 * i + l16;
      if (m >= M) m = M - 1;
      tf[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(T + m * 32 + 8 * q));
    }
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      int64_t n = n0 + wn * kWC + 16 * j + l16;
      if (n >= N) n = N - 1;
      uint16_t u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = Lu[(int64_t)(8 * q + e) * N + n];
      lf[j] = __builtin_bit_cast(v8bf, u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kNJ; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lf[j], tf[i], acc[i][j], 0, 0, 0);
  }

  // lane (l16, q) holds columns n0 + 48 wn + 16 j + 4 q + (0..3) of row m0 + 64 wm + 16 i + l16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + wm * 64 + 16 * i + l16;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < kNJ; ++j) {
      const int64_t n = n0 + wn * kWC + 16 * j + 4 * q;
      if (n >= N) continue;                         // N % 16 == 0: a lane's 4 columns are all in or all out
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (bias) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32(bias[n + e]);
      }
      const uint32_t lo = bf16x2_rne(v[0], v[1]);
      const uint32_t hi = bf16x2_rne(v[2], v[3]);
      *reinterpret_cast<uint2*>(D + row * ldd + n) = make_uint2(lo, hi);
    }
  }
}

// workspace: A and B dequantized to fp16 ([M][K], [N][K]), then with the low-rank
// branch T [M][32] bf16; every part 256-byte aligned
namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

size_t w4a4_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank) {
  size_t b = align256((size_t)M * K * 2) + align256((size_t)N * K * 2);
  if (rank > 0) b += align256((size_t)M * 32 * 2);
  return b;
}

hipError_t launch_lowrank_t(int64_t M, int64_t K, const uint16_t* x_bf16, const uint16_t* l_down, uint16_t* T,
                            hipStream_t st) {
  const int64_t blocks = (M + 15) / 16;
  trace_launch(kInfoW4a4LowRank, dim3((unsigned)blocks), "M=%lld K=%lld rank=32", (long long)M, (long long)K);
  hipLaunchKernelGGL(w4a4_lowrank_kernel, dim3((unsigned)blocks), dim3(64 * kLrWavesAlone), 0, st, x_bf16, l_down, T,
                     M, K);
  return hipGetLastError();
}

const KernelInfo kInfoW4a4Prep = {"w4a4_prep_kernel", "fgg_scaled_gemm (W4A4)", 16, 32, 0, 256, 0, 0,
                                  kLrWaves * 32 * 32 * 2 + kLrWaves * 2 * 64 * 16,
                                  kLrWaves * 32 * 32 * 2 + kLrWaves * 2 * 64 * 16, (const void*)w4a4_prep_kernel};
const KernelInfo kInfoW4a4LowRank = {"w4a4_lowrank_kernel", "fgg_scaled_gemm (MXFP4 low-rank branch)", 16, 32, 0,
                                     64 * kLrWavesAlone, 0, 0,
                                     kLrWavesAlone * 32 * 32 * 2 + kLrWavesAlone * 2 * 64 * 16,
                                     kLrWavesAlone * 32 * 32 * 2 + kLrWavesAlone * 2 * 64 * 16,
                                     (const void*)w4a4_lowrank_kernel};
const KernelInfo kInfoW4a4Gemm = {"w4a4_gemm_kernel", "fgg_scaled_gemm (W4A4)", w4::BM, w4::BN, w4::BK,
                                  64 * w4::kWaves, w4::kStages, w4::kStageBytes, 0, w4::kStages * w4::kStageBytes,
                                  (const void*)w4a4_gemm_kernel};

hipError_t launch_w4a4(int64_t M, int64_t N, int64_t K, const uint8_t* a, const float* sa,
                       const uint8_t* b, const float* sb, const uint16_t* x_bf16,
                       const uint16_t* l_down, const uint16_t* l_up, int32_t rank,
                       const uint16_t* bias, uint16_t* d, int64_t ldd, void* ws, int num_cus, hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  if (M % 128 != 0 || N % 128 != 0 || K % 128 != 0 || K == 0) return hipErrorInvalidValue;
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  uint16_t* Ah = reinterpret_cast<uint16_t*>(w);
  uint16_t* Bh = reinterpret_cast<uint16_t*>(w + align256((size_t)M * K * 2));
  uint8_t* rest = w + align256((size_t)M * K * 2) + align256((size_t)N * K * 2);
  (void)num_cus;
  const int64_t na = M * K / 8, nb = N * K / 8;
  uint16_t* T = reinterpret_cast<uint16_t*>(rest);
  const int64_t per = 256 * kItems;
  const int64_t lr_blocks = rank > 0 ? (M + 15) / 16 : 0;
  const int64_t blocks = lr_blocks + (na + per - 1) / per + (nb + per - 1) / per;
  trace_launch(kInfoW4a4Prep, dim3((unsigned)blocks), "M=%lld N=%lld K=%lld rank=%d (%lld low-rank blocks)",
               (long long)M, (long long)N, (long long)K, (int)rank, (long long)lr_blocks);
  hipLaunchKernelGGL(w4a4_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, sa, na, Ah, b, sb, nb, Bh,
                     x_bf16, l_down, rank > 0 ? T : nullptr, M, K, lr_blocks);
  const int64_t tiles = ((M + w4::BM - 1) / w4::BM) * ((N + w4::BN - 1) / w4::BN);
  const int64_t grid = (tiles + 7) / 8 * 8;          // a multiple of the XCD count (tile order above)
  trace_launch(kInfoW4a4Gemm, dim3((unsigned)grid), "M=%lld N=%lld K=%lld%s", (long long)M, (long long)N,
               (long long)K, bias ? " bias" : "");
  hipLaunchKernelGGL(w4a4_gemm_kernel, dim3((unsigned)grid), dim3(64 * w4::kWaves), 0, st, M, N, K, Ah, Bh,
                     rank > 0 ? T : nullptr, l_up, (int)rank, bias, d, ldd);
  return hipGetLastError();
}

}  // namespace fgg
