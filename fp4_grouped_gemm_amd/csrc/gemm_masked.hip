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
// each K block's partial product is promoted with one FMA per output.
//
// FP4 weights (the decode path): gemm_masked_fp4_lds_kernel, eight waves per
// workgroup, each streaming 16 weight rows, the activations shared through
// LDS.  e4m3 weights: gemm_masked_v2_kernel, activations read per wave.
//
// Tiled FP4 weights (FGG_E2M1X2_TILED, written by pack_fp4_tiles_kernel): the
// interleaved storage the FP4 tensor-core path wants ([FP4MoE] §2.1 FP4 data
// aligned to 128-bit boundaries in an interleaved layout, §3.1 a dedicated
// packed weight format).  Here the interleave is the MFMA operand itself:
// each 16-row x 128-K tile is 1 KB in lane order (lane 16c + r holds row r,
// K [32c, 32c+32)), so a wave's weight load of one K block is one contiguous
// 1 KB; the E8M0 scales of a 16-row group are 256 bytes per 4 K blocks (row r:
// its 16 scale bytes).  Measured: the plain layout (16 rows x 64 B per load)
// streams at ~4.8 TB/s, the tiled one at ~5.7 TB/s.
#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

// Streaming variant: each wave owns 16*NT weight rows (columns of D) over all
// of K, so its weight bytes are NT runs of 16 consecutive rows (one
// contiguous block of 16*K/2 bytes each).  Loads are double-buffered in
// registers: the loads of K blocks [kb0+U, kb0+2U) are in flight while the
// MFMAs of [kb0, kb0+U) run.  The E8M0 scales of 4 K blocks of a row are one
// 16-byte load (the four lanes of a row share it); lane group q picks its
// 32-block's byte with a bit-field extract.  Accumulation order per output is
// the same as gemm_masked_kernel's (K blocks in increasing order).
template <bool B_FP4, int NT, int U>
struct MaskedStage {
  v8i a[U];
  float sa[U];
  uint4 b[U][NT];
  uint4 lo_hi[B_FP4 ? 1 : U][NT];            // fp8 weights: bytes 64..127 of the K block
  uint32_t sc[NT][B_FP4 ? (U + 3) / 4 * 4 : U];   // FP4: scale dwords; fp8: fp32 bits per K block
};

template <bool B_FP4, int NT, int U, bool PF>
__global__ void __launch_bounds__(256)
gemm_masked_v2_kernel(int G, int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
                      const float* __restrict__ SA, const uint8_t* __restrict__ B, const void* __restrict__ SBv,
                      const int32_t* __restrict__ masked_m, uint16_t* __restrict__ D, int64_t ldd) {
  static_assert(U % 4 == 0, "U must be a multiple of 4");
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t waves_per_group = N / (16 * NT);
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)G * waves_per_group) return;
  const int g = (int)(wid / waves_per_group);
  const int64_t n_base = (wid % waves_per_group) * 16 * NT;
  int mm = masked_m[g];
  mm = mm < 0 ? 0 : (mm > (int)M ? (int)M : mm);
  if (mm == 0) return;
  const int nkb = (int)(K / 128);
  const bool row_live = l16 < mm;
  const uint8_t* Ar = A + ((int64_t)g * M + l16) * K;
  const float* SAr = SA + (int64_t)g * nkb * M + l16;
  const int64_t brow_bytes = B_FP4 ? K / 2 : K;
  const uint8_t* Br = B + ((int64_t)g * N + n_base + l16) * brow_bytes;
  const uint8_t* Sr8 = reinterpret_cast<const uint8_t*>(SBv) + ((int64_t)g * N + n_base + l16) * (K / 32);
  const float* Sf = reinterpret_cast<const float*>(SBv) + ((int64_t)g * (N / 128) + n_base / 128) * nkb;

  auto load = [&](MaskedStage<B_FP4, NT, U>& st, int kb0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u;
      if (kb < nkb) {
        if (row_live) {
          const uint4 lo = *reinterpret_cast<const uint4*>(Ar + (int64_t)kb * 128 + 16 * q);
          const uint4 hi = *reinterpret_cast<const uint4*>(Ar + (int64_t)kb * 128 + 64 + 16 * q);
          st.a[u] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          st.sa[u] = SAr[(int64_t)kb * M];
        } else {
          st.a[u] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          st.sa[u] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const uint8_t* br = Br + (int64_t)(16 * j) * brow_bytes;
          if (B_FP4) {
            st.b[u][j] = *reinterpret_cast<const uint4*>(br + (int64_t)kb * 64 + 16 * q);
          } else {
            st.b[u][j] = *reinterpret_cast<const uint4*>(br + (int64_t)kb * 128 + 16 * q);
            st.lo_hi[B_FP4 ? 0 : u][j] = *reinterpret_cast<const uint4*>(br + (int64_t)kb * 128 + 64 + 16 * q);
            st.sc[j][u] = __float_as_uint(Sf[((16 * j + 0) / 128) * nkb + kb]);
          }
        }
      }
    }
    if (B_FP4) {
#pragma unroll
      for (int u4 = 0; u4 < U / 4; ++u4) {
        const int kb = kb0 + 4 * u4;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const uint8_t* sr = Sr8 + (int64_t)(16 * j) * (K / 32) + (int64_t)kb * 4;
          if (kb + 4 <= nkb) {
            const uint4 v = *reinterpret_cast<const uint4*>(sr);
            st.sc[j][4 * u4 + 0] = v.x; st.sc[j][4 * u4 + 1] = v.y;
            st.sc[j][4 * u4 + 2] = v.z; st.sc[j][4 * u4 + 3] = v.w;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              st.sc[j][4 * u4 + i] = kb + i < nkb ? *reinterpret_cast<const uint32_t*>(sr + 4 * i) : 0x7F7F7F7Fu;
          }
        }
      }
    }
  };

  v4f acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const MaskedStage<B_FP4, NT, U>& st, int kb0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb0 + u >= nkb) break;   // wave-uniform
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        v4f p;
        float s;
        if (B_FP4) {
          const v8i bf = v8i{(int)st.b[u][j].x, (int)st.b[u][j].y, (int)st.b[u][j].z, (int)st.b[u][j].w, 0, 0, 0, 0};
          const int sc = (int)__builtin_amdgcn_ubfe(st.sc[j][u], 8 * q, 8);
          p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, st.a[u], v4f{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, sc, 0, 127);
          s = st.sa[u];
        } else {
          const uint4 lo = st.b[u][j], hi = st.lo_hi[B_FP4 ? 0 : u][j];
          const v8i bf = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
          p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, st.a[u], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
          s = st.sa[u] * __uint_as_float(st.sc[j][u]);
        }
        acc[j][0] = fmaf(p[0], s, acc[j][0]);
        acc[j][1] = fmaf(p[1], s, acc[j][1]);
        acc[j][2] = fmaf(p[2], s, acc[j][2]);
        acc[j][3] = fmaf(p[3], s, acc[j][3]);
      }
    }
  };

  if (PF) {
    MaskedStage<B_FP4, NT, U> s0, s1;
    load(s0, 0);
    for (int kb0 = 0; kb0 < nkb; kb0 += 2 * U) {
      if (kb0 + U < nkb) load(s1, kb0 + U);
      compute(s0, kb0);
      if (kb0 + U >= nkb) break;
      if (kb0 + 2 * U < nkb) load(s0, kb0 + 2 * U);
      compute(s1, kb0 + U);
    }
  } else {
    MaskedStage<B_FP4, NT, U> s0;
    for (int kb0 = 0; kb0 < nkb; kb0 += U) {
      load(s0, kb0);
      compute(s0, kb0);
    }
  }
  if (!row_live) return;
  uint16_t* drow = D + ((int64_t)g * M + l16) * ldd + n_base + 4 * q;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const uint32_t lo = bf16x2_rne(acc[j][0], acc[j][1]);
    const uint32_t hi = bf16x2_rne(acc[j][2], acc[j][3]);
    *reinterpret_cast<uint2*>(drow + 16 * j) = make_uint2(lo, hi);
  }
}

// FP4-weight decode kernel with the activations shared through LDS.  A
// workgroup of W waves covers 16*W consecutive weight rows of one group; each
// wave streams its own 16 rows (16 rows x K/2 bytes, one contiguous block)
// U K blocks per step, with the next step's weight bytes and E8M0 scales
// loaded into registers while the current step's MFMAs run.  The group's
// activation rows and their 1x128 scales are loaded once per workgroup, UA K
// blocks at a time, into a double-buffered LDS chunk [16 rows][UA*128 bytes]
// (rows padded by 32 bytes: gfx950 serves a ds_read_b128 in cycles of 16 lanes
// mixing two lane groups q, lanes {0-3, 12-15, 20-23, 24-27} (+32) and {4-11, 16-19,
// 28-31} (+32) (measured), and with a row stride of 34 16-byte slots row r of group q
// sits on slot 2r + q (mod 16): distinct within every cycle; the former 16-byte pad
// put two lanes on one slot and doubled each read); the next chunk's global loads are in
// flight during the current chunk, and one barrier per chunk publishes it.
// 16 bytes at p (16-byte aligned) with the nontemporal (streaming) cache policy.
__device__ inline uint4 load_stream16(const uint8_t* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int UA>
struct MaskedLds {
  static constexpr int kRowBytes = UA * 128 + 32;
  static constexpr int kABytes = 16 * kRowBytes;
  static constexpr int kBufBytes = kABytes + UA * 16 * 4;   // + sa[UA][16]
  static constexpr int kBytes = 2 * kBufBytes;
};

template <int U, int UA, int W, bool TILED>
__global__ void __launch_bounds__(64 * W)
gemm_masked_fp4_lds_kernel(int G, int64_t M, int64_t N, int64_t K, const uint8_t* __restrict__ A,
                           const float* __restrict__ SA, const uint8_t* __restrict__ B,
                           const uint8_t* __restrict__ SB, const int32_t* __restrict__ masked_m,
                           uint16_t* __restrict__ D, int64_t ldd) {
  static_assert(U % 4 == 0 && UA % U == 0, "U must be a multiple of 4 and divide UA");
  using L = MaskedLds<UA>;
  constexpr int kSPC = UA / U;   // weight steps per activation chunk
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t wg_per_group = N / (16 * W);
  const int g = (int)(blockIdx.x / wg_per_group);
  const int64_t n_base = (blockIdx.x % wg_per_group) * 16 * W + 16 * wave;
  int mm = masked_m[g];
  mm = mm < 0 ? 0 : (mm > (int)M ? (int)M : mm);
  if (mm == 0) return;                     // whole workgroup (uniform)
  const int nkb = (int)(K / 128);
  const int nsteps = (nkb + U - 1) / U;
  const int nchunks = (nkb + UA - 1) / UA;
  const uint8_t* Ag = A + (int64_t)g * M * K;
  const float* SAg = SA + (int64_t)g * nkb * M;
  // this lane's weight bytes of K block kb: Br + kb * kBStride; its row's scale bytes of
  // K blocks [kb, kb + 4) (kb a multiple of 4): Sr + (kb / 4) * kSStride
  const int64_t nspan = (nkb + 3) / 4;
  const uint8_t* Br = TILED ? B + (((int64_t)g * (N / 16) + n_base / 16) * nkb) * 1024 + lane * 16
                            : B + ((int64_t)g * N + n_base + l16) * (K / 2) + 16 * q;
  const uint8_t* Sr = TILED ? SB + (((int64_t)g * (N / 16) + n_base / 16) * nspan) * 256 + l16 * 16
                            : SB + ((int64_t)g * N + n_base + l16) * (K / 32);
  constexpr int64_t kBStride = TILED ? 1024 : 64;
  constexpr int64_t kSStride = TILED ? 256 : 16;

  // one activation chunk: 16 rows x UA*128 bytes = UA*128 pieces of 16 bytes
  constexpr int kAPieces = 16 * UA * 8;
  constexpr int kAPer = (kAPieces + 64 * W - 1) / (64 * W);
  constexpr int kSPer = (UA * 16 + 64 * W - 1) / (64 * W);
  uint4 areg[kAPer];
  float sareg[kSPer];
  auto load_a = [&](int c) {
    const int kb0 = c * UA;
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int piece = tid + 64 * W * i;
      const int row = piece / (UA * 8), col = piece % (UA * 8);
      if (piece < kAPieces && row < mm && kb0 + col / 8 < nkb)
        areg[i] = *reinterpret_cast<const uint4*>(Ag + (int64_t)row * K + (int64_t)kb0 * 128 + 16 * col);
    }
#pragma unroll
    for (int i = 0; i < kSPer; ++i) {
      const int e = tid + 64 * W * i, u = e / 16, m = e % 16;
      if (e < UA * 16) sareg[i] = (m < mm && kb0 + u < nkb) ? SAg[(int64_t)(kb0 + u) * M + m] : 0.0f;
    }
  };
  auto store_a = [&](int buf) {
    uint8_t* base = lds + buf * L::kBufBytes;
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int piece = tid + 64 * W * i;
      const int row = piece / (UA * 8), col = piece % (UA * 8);
      if (piece < kAPieces && row < mm)
        *reinterpret_cast<uint4*>(base + row * L::kRowBytes + 16 * col) = areg[i];
    }
#pragma unroll
    for (int i = 0; i < kSPer; ++i) {
      const int e = tid + 64 * W * i;
      if (e < UA * 16) reinterpret_cast<float*>(base + L::kABytes)[e] = sareg[i];
    }
  };

  struct BStage {
    uint4 b[U];
    uint32_t sc[U];
  };
  // Weight bytes are read exactly once: nontemporal loads (streaming cache policy) keep
  // them from displacing the activations, which every workgroup of a group re-reads
  // (measured: 87.5-90 us -> 81.5 us for the 499 MB decode stream).
  auto load_b = [&](BStage& st, int step) {
    const int kb0 = step * U;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (kb0 + u < nkb) st.b[u] = load_stream16(Br + (int64_t)(kb0 + u) * kBStride);
#pragma unroll
    for (int u4 = 0; u4 < U / 4; ++u4) {
      const int kb = kb0 + 4 * u4;
      const uint8_t* sr = Sr + (int64_t)(kb / 4) * kSStride;
      if (TILED || kb + 4 <= nkb) {         // (a tiled span is always 16 bytes, padded with 2^0)
        const uint4 v = load_stream16(sr);
        st.sc[4 * u4 + 0] = v.x; st.sc[4 * u4 + 1] = v.y; st.sc[4 * u4 + 2] = v.z; st.sc[4 * u4 + 3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st.sc[4 * u4 + i] = kb + i < nkb ? *reinterpret_cast<const uint32_t*>(sr + 4 * i) : 0x7F7F7F7Fu;
      }
    }
  };

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const BStage& st, int step) {
    const int kb0 = step * U;
    const int c = kb0 / UA;
    const uint8_t* base = lds + (c & 1) * L::kBufBytes;
    const uint8_t* arow = base + l16 * L::kRowBytes + 16 * q + (kb0 - c * UA) * 128;
    const float* sa = reinterpret_cast<const float*>(base + L::kABytes) + (kb0 - c * UA) * 16 + l16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb0 + u >= nkb) break;   // uniform
      const uint4 lo = *reinterpret_cast<const uint4*>(arow + u * 128);
      const uint4 hi = *reinterpret_cast<const uint4*>(arow + u * 128 + 64);
      const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      const v8i bf = v8i{(int)st.b[u].x, (int)st.b[u].y, (int)st.b[u].z, (int)st.b[u].w, 0, 0, 0, 0};
      const int sc = (int)__builtin_amdgcn_ubfe(st.sc[u], 8 * q, 8);
      const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, v4f{0.f, 0.f, 0.f, 0.f}, 4, 0, 0, sc,
                                                                      0, 127);
      const float s = sa[u * 16];
      acc[0] = fmaf(p[0], s, acc[0]);
      acc[1] = fmaf(p[1], s, acc[1]);
      acc[2] = fmaf(p[2], s, acc[2]);
      acc[3] = fmaf(p[3], s, acc[3]);
    }
  };
  // Around a weight step: at the first step of chunk c the loads of chunk c+1
  // are issued; after the last step of chunk c they are stored into buffer
  // (c+1)&1 (last read during chunk c-1, before the previous barrier) and a
  // barrier publishes them.
  auto step_body = [&](BStage& cur, BStage& nxt, int step) {
    const int c = step / kSPC, within = step - c * kSPC;
    const bool more = c + 1 < nchunks;
    if (within == 0 && more) load_a(c + 1);
    if (step + 1 < nsteps) load_b(nxt, step + 1);
    compute(cur, step);
    if ((within == kSPC - 1 || step == nsteps - 1) && more) {
      store_a((c + 1) & 1);
      __syncthreads();
    }
  };

  BStage s0, s1;
  load_a(0);
  load_b(s0, 0);
  store_a(0);
  __syncthreads();
  for (int step = 0; step < nsteps; step += 2) {
    step_body(s0, s1, step);
    if (step + 1 >= nsteps) break;
    step_body(s1, s0, step + 1);
  }
  if (l16 >= mm) return;
  uint16_t* drow = D + ((int64_t)g * M + l16) * ldd + n_base + 4 * q;
  const uint32_t lo = bf16x2_rne(acc[0], acc[1]);
  const uint32_t hi = bf16x2_rne(acc[2], acc[3]);
  *reinterpret_cast<uint2*>(drow) = make_uint2(lo, hi);
}

const KernelInfo kInfoMaskedFp4Tiled = {
    "gemm_masked_fp4_lds_kernel<tiled>", "fgg_grouped_gemm_scaled (masked, E2M1X2_TILED + E8M0/32)", 16, 128, 512,
    512, 2, MaskedLds<4>::kBufBytes, 0, MaskedLds<4>::kBytes, (const void*)gemm_masked_fp4_lds_kernel<4, 4, 8, true>};
const KernelInfo kInfoMaskedFp4 = {
    "gemm_masked_fp4_lds_kernel<plain>", "fgg_grouped_gemm_scaled (masked, E2M1X2 + E8M0/32)", 16, 128, 512, 512, 2,
    MaskedLds<4>::kBufBytes, 0, MaskedLds<4>::kBytes, (const void*)gemm_masked_fp4_lds_kernel<4, 4, 8, false>};
const KernelInfo kInfoMaskedFp8 = {"gemm_masked_v2_kernel<e4m3>", "fgg_grouped_gemm_scaled (masked, e4m3 128x128)",
                                   16, 128, 512, 256, 0, 0, 0, 0,
                                   (const void*)gemm_masked_v2_kernel<false, 2, 4, true>};

hipError_t launch_gemm_masked(bool b_fp4, bool tiled, int32_t G, int64_t M, int64_t N, int64_t K,
                              const uint8_t* a, const float* sa, const uint8_t* b, const void* sb,
                              const int32_t* masked_m, uint16_t* d, int64_t ldd, hipStream_t st) {
  if (N % 128 != 0 || M > 16 || (tiled && !b_fp4)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((int64_t)G * (N / 128)));
  trace_launch(b_fp4 ? (tiled ? kInfoMaskedFp4Tiled : kInfoMaskedFp4) : kInfoMaskedFp8, grid,
               "G=%d M=%lld N=%lld K=%lld", (int)G, (long long)M, (long long)N, (long long)K);
  if (b_fp4 && tiled) {
    // 8 waves x 16 weight rows per workgroup, 4 K blocks per step and per activation chunk
    hipLaunchKernelGGL((gemm_masked_fp4_lds_kernel<4, 4, 8, true>), grid, dim3(512), 0, st, G, M, N, K, a, sa, b,
                       reinterpret_cast<const uint8_t*>(sb), masked_m, d, ldd);
  } else if (b_fp4) {
    hipLaunchKernelGGL((gemm_masked_fp4_lds_kernel<4, 4, 8, false>), grid, dim3(512), 0, st, G, M, N, K, a, sa, b,
                       reinterpret_cast<const uint8_t*>(sb), masked_m, d, ldd);
  } else {
    // 4 waves x 32 weight rows per workgroup
    hipLaunchKernelGGL((gemm_masked_v2_kernel<false, 2, 4, true>), grid, dim3(256), 0, st, G, M, N, K, a, sa, b,
                       sb, masked_m, d, ldd);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP4 weight tiling (offline): [G][N][K/2] codes and [G][N][K/32] E8M0 scales to
// the tiled layout read by the decode kernel above.  A pure byte permutation.
//   codes: tile (g, n/16, kb) is 1 KB; its 16-byte piece 16c + r is row 16(n/16) + r,
//          bytes [64 kb + 16 c, 64 kb + 16 c + 16) of that row
//   scales: span (g, n/16, j/16) is 256 bytes; bytes [16 r, 16 r + 16) are row
//          16(n/16) + r's scale bytes [16 (j/16), 16 (j/16) + 16), 127 past K/32
__global__ void __launch_bounds__(256)
pack_fp4_tiles_kernel(const uint8_t* __restrict__ b, uint8_t* __restrict__ bt, int64_t pieces, int64_t K) {
  const int64_t nkb = K / 128;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < pieces; p += (int64_t)gridDim.x * 256) {
    const int lane = (int)(p & 63);
    const int64_t tile = p >> 6;                       // (g * N/16 + nb) * nkb + kb
    const int64_t kb = tile % nkb, gnb = tile / nkb;   // gnb = g * N/16 + nb
    const int r = lane & 15, c = lane >> 4;
    const int64_t row = gnb * 16 + r;                  // = g * N + 16 nb + r
    *reinterpret_cast<uint4*>(bt + p * 16) = *reinterpret_cast<const uint4*>(b + row * (K / 2) + kb * 64 + c * 16);
  }
}

__global__ void __launch_bounds__(256)
pack_fp4_scale_tiles_kernel(const uint8_t* __restrict__ s, uint8_t* __restrict__ st, int64_t rows_spans,
                            int64_t K) {
  const int64_t nsc = K / 32, nspan = (nsc + 15) / 16;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows_spans; i += (int64_t)gridDim.x * 256) {
    // i = ((g * N/16 + nb) * nspan + span) * 16 + r
    const int r = (int)(i & 15);
    const int64_t t = i >> 4, span = t % nspan, gnb = t / nspan;
    const uint8_t* src = s + (gnb * 16 + r) * nsc + span * 16;
    uint8_t v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = span * 16 + e < nsc ? src[e] : (uint8_t)127;
    uint4 w;
    w.x = (uint32_t)v[0] | ((uint32_t)v[1] << 8) | ((uint32_t)v[2] << 16) | ((uint32_t)v[3] << 24);
    w.y = (uint32_t)v[4] | ((uint32_t)v[5] << 8) | ((uint32_t)v[6] << 16) | ((uint32_t)v[7] << 24);
    w.z = (uint32_t)v[8] | ((uint32_t)v[9] << 8) | ((uint32_t)v[10] << 16) | ((uint32_t)v[11] << 24);
    w.w = (uint32_t)v[12] | ((uint32_t)v[13] << 8) | ((uint32_t)v[14] << 16) | ((uint32_t)v[15] << 24);
    *reinterpret_cast<uint4*>(st + i * 16) = w;
  }
}

const KernelInfo kInfoPackFp4 = {"pack_fp4_tiles_kernel", "fgg_pack_fp4_weights", 0, 0, 0, 256, 0, 0, 0, 0,
                                 (const void*)pack_fp4_tiles_kernel};
const KernelInfo kInfoPackFp4Scales = {"pack_fp4_scale_tiles_kernel", "fgg_pack_fp4_weights", 0, 0, 0, 256, 0, 0, 0,
                                       0, (const void*)pack_fp4_scale_tiles_kernel};

void fp4_tiled_bytes(int32_t G, int64_t N, int64_t K, size_t* b_bytes, size_t* s_bytes) {
  *b_bytes = (size_t)G * (size_t)N * (size_t)(K / 2);
  *s_bytes = (size_t)G * (size_t)(N / 16) * (size_t)((K / 32 + 15) / 16) * 256;
}

hipError_t launch_pack_fp4(int32_t G, int64_t N, int64_t K, const uint8_t* b, const uint8_t* s, uint8_t* bt,
                           uint8_t* st, int num_cus, hipStream_t stream) {
  if (N % 16 != 0 || K % 128 != 0) return hipErrorInvalidValue;
  if (G == 0 || N == 0 || K == 0) return hipSuccess;
  const int64_t pieces = (int64_t)G * N * (K / 128) * 4;          // 16-byte pieces of the codes
  const int64_t rows_spans = (int64_t)G * N * ((K / 32 + 15) / 16);
  const int64_t cap = (int64_t)num_cus * 16;
  int64_t g1 = (pieces + 255) / 256, g2 = (rows_spans + 255) / 256;
  if (g1 > cap) g1 = cap;
  if (g2 > cap) g2 = cap;
  trace_launch(kInfoPackFp4, dim3((unsigned)g1), "G=%d N=%lld K=%lld", (int)G, (long long)N, (long long)K);
  trace_launch(kInfoPackFp4Scales, dim3((unsigned)g2), "G=%d N=%lld K=%lld", (int)G, (long long)N, (long long)K);
  hipLaunchKernelGGL(pack_fp4_tiles_kernel, dim3((unsigned)g1), dim3(256), 0, stream, b, bt, pieces, K);
  hipLaunchKernelGGL(pack_fp4_scale_tiles_kernel, dim3((unsigned)g2), dim3(256), 0, stream, s, st, rows_spans, K);
  return hipGetLastError();
}

}  // namespace fgg
