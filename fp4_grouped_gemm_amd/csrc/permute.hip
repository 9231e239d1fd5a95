// MoE routing glue: stable padded counting sort of (token, slot) pairs into
// per-expert row segments, the gather of quantized rows into that order, and
// the gate-weighted combine back to token order.
//
// [DeepGEMM] bhfrc.com/news/60438 §5.3: the grouped GEMM needs each group's
// id and token offsets, with every expert's rows contiguous.  [FP4MoE]
// "Blackwell架构下FP4 MoE模型的TFLOPS性能优化" §4.2: expert group sizes are
// multiples of 128.  [MegaMoE] www.mqxn.cn/news/59821 §1, §3: the layer
// output is the gate-weighted sum of the selected experts' outputs.
//
// Pipeline (all integer work, deterministic):
//   hist:    block b counts its CHUNK pairs per expert (LDS atomics).
//   scan:    one block: per expert, exclusive prefix over blocks -> base[b][e];
//            padded counts -> offsets (exclusive scan over experts).
//   scatter: block b walks its pairs in order; a pair's rank among equal
//            experts comes from wave ballots (stable), plus per-wave and
//            per-block running counts.
//   gather:  rows [0, M_total) copy their token's codes and scales (zeros
//            for padding rows).
#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

static constexpr int kChunk = 1024;   // pairs per block in hist/scatter
static constexpr int kMaxE = 1024;

size_t permute_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  const int64_t pairs = T * (int64_t)k;
  const int64_t nblk = (pairs + kChunk - 1) / kChunk;
  return (size_t)(2 * nblk * (int64_t)E * sizeof(int32_t)) + 256;
}

__device__ inline int valid_expert(int e, int E) { return (e >= 0 && e < E) ? e : -1; }

__global__ void __launch_bounds__(256) permute_hist_kernel(const int32_t* __restrict__ ids, int64_t pairs,
                                                            int E, int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxE];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += 256) {
    const int64_t p = p0 + i;
    if (p < pairs) {
      const int e = valid_expert(ids[p], E);
      if (e >= 0) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One block of 1024 threads; thread e owns expert e.
__global__ void __launch_bounds__(1024) permute_scan_kernel(int32_t* __restrict__ hist, int64_t nblk, int E,
                                                             int align, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ counts) {
  __shared__ int scan[kMaxE];
  const int e = threadIdx.x;
  int running = 0;
  if (e < E) {
    for (int64_t b = 0; b < nblk; ++b) {
      const int h = hist[b * E + e];
      hist[b * E + e] = running;        // exclusive prefix over blocks (made absolute below)
      running += h;
    }
    counts[e] = running;
  }
  const int padded = (e < E) ? ((running + align - 1) / align) * align : 0;
  scan[e] = padded;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 entries
  for (int off = 1; off < kMaxE; off <<= 1) {
    const int v = (e >= off) ? scan[e - off] : 0;
    __syncthreads();
    scan[e] += v;
    __syncthreads();
  }
  const int excl = scan[e] - padded;
  if (e < E) {
    offsets[e] = excl;
    for (int64_t b = 0; b < nblk; ++b) hist[b * E + e] += excl;
  }
  if (e == E - 1) offsets[E] = scan[e];
}

__global__ void __launch_bounds__(256) fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

__global__ void __launch_bounds__(256) permute_scatter_kernel(const int32_t* __restrict__ ids, int64_t pairs,
                                                               int E, const int32_t* __restrict__ base,
                                                               int32_t* __restrict__ src_to_row,
                                                               int32_t* __restrict__ row_to_src, int64_t M_cap) {
  __shared__ int running[kMaxE];
  __shared__ int wave_cnt[4][kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += 256) {
    running[e] = base[(int64_t)blockIdx.x * E + e];
    wave_cnt[0][e] = wave_cnt[1][e] = wave_cnt[2][e] = wave_cnt[3][e] = 0;
  }
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kChunk;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int sub = 0; sub < kChunk / 256; ++sub) {
    const int64_t p = p0 + sub * 256 + threadIdx.x;
    const int e = (p < pairs) ? valid_expert(ids[p], E) : -1;
    // rank among lower lanes of this wave with the same expert
    int rank = 0;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int el = __shfl(e, leader);
      const uint64_t same = __ballot(e == el);
      if (e == el) rank = __popcll(same & lt_mask);
      if (lane == leader) wave_cnt[wave][el] = __popcll(same);
      todo &= ~same;
    }
    __syncthreads();
    if (e >= 0) {
      int before = running[e] + rank;
      for (int w = 0; w < wave; ++w) before += wave_cnt[w][e];
      src_to_row[p] = before;
      if (before < M_cap) row_to_src[before] = (int32_t)p;
    } else if (p < pairs) {
      src_to_row[p] = -1;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += 256) {
      running[x] += wave_cnt[0][x] + wave_cnt[1][x] + wave_cnt[2][x] + wave_cnt[3][x];
      wave_cnt[0][x] = wave_cnt[1][x] = wave_cnt[2][x] = wave_cnt[3][x] = 0;
    }
    __syncthreads();
  }
}

// Copy each row's token codes (K bytes) and 1x128 scales; zeros for padding.
__global__ void __launch_bounds__(256) permute_gather_kernel(const int32_t* __restrict__ offsets, int E, int k,
                                                              const int32_t* __restrict__ row_to_src,
                                                              const uint8_t* __restrict__ xq,
                                                              const float* __restrict__ xs, int64_t T,
                                                              int64_t K, uint8_t* __restrict__ a_out,
                                                              float* __restrict__ sa_out, int64_t M_cap) {
  int64_t m_total = offsets[E];
  if (m_total > M_cap) m_total = M_cap;
  const int64_t nkb = K / 128;
  for (int64_t r = blockIdx.x; r < m_total; r += gridDim.x) {
    const int32_t p = row_to_src[r];
    uint4* dst = reinterpret_cast<uint4*>(a_out + r * K);
    if (p >= 0) {
      const int64_t t = p / k;
      const uint4* src = reinterpret_cast<const uint4*>(xq + t * K);
      for (int64_t i = threadIdx.x; i < K / 16; i += 256) dst[i] = src[i];
      for (int64_t kb = threadIdx.x; kb < nkb; kb += 256) sa_out[kb * M_cap + r] = xs[kb * T + t];
    } else {
      for (int64_t i = threadIdx.x; i < K / 16; i += 256) dst[i] = make_uint4(0, 0, 0, 0);
      for (int64_t kb = threadIdx.x; kb < nkb; kb += 256) sa_out[kb * M_cap + r] = 0.0f;
    }
  }
}

hipError_t launch_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t align,
                          const uint8_t* xq, const float* xs, int64_t K, int32_t* offsets,
                          int32_t* counts, int32_t* src_to_row, int32_t* row_to_src, uint8_t* a_out,
                          float* sa_out, int64_t M_cap, void* ws, hipStream_t st) {
  const int64_t pairs = T * (int64_t)k;
  if (pairs == 0) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, offsets, (int64_t)E + 1, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, counts, (int64_t)E, 0);
    if (M_cap > 0)
      hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((M_cap + 255) / 256 < 1024 ? (M_cap + 255) / 256 : 1024)), dim3(256), 0, st, row_to_src, M_cap, -1);
    return hipGetLastError();
  }
  const int64_t nblk = (pairs + kChunk - 1) / kChunk;
  int32_t* hist = reinterpret_cast<int32_t*>(ws);
  hipLaunchKernelGGL(permute_hist_kernel, dim3((unsigned)nblk), dim3(256), 0, st, ids, pairs, (int)E, hist);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, st, hist, nblk, (int)E, (int)align, offsets, counts);
  if (M_cap > 0) {
    const int64_t g = (M_cap + 255) / 256;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)(g < 2048 ? g : 2048)), dim3(256), 0, st, row_to_src, M_cap, -1);
  }
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)nblk), dim3(256), 0, st, ids, pairs, (int)E, hist,
                     src_to_row, row_to_src, M_cap);
  if (xq != nullptr && M_cap > 0) {
    hipLaunchKernelGGL(permute_gather_kernel, dim3(2048), dim3(256), 0, st, offsets, (int)E, (int)k, row_to_src,
                       xq, xs, T, K, a_out, sa_out, M_cap);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: one 256-thread block per token; each thread owns 8 columns (16 B)
// at a time and sums the routed slots in increasing j, fp32 FMA.
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ y, int64_t ldy,
                                                       const int32_t* __restrict__ src_to_row,
                                                       const float* __restrict__ w, int64_t T, int k,
                                                       int64_t N, uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t t = blockIdx.x;
  for (int64_t n0 = (int64_t)threadIdx.x * 8; n0 < N; n0 += 256 * 8) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const int32_t row = src_to_row[t * k + j];
      if (row < 0) continue;
      const float wj = w[t * k + j];
      const uint4 u = *reinterpret_cast<const uint4*>(y + (int64_t)row * ldy + n0);
      const uint32_t q[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wj, bf16_to_f32((uint16_t)(q[i] & 0xFFFFu)), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj, bf16_to_f32((uint16_t)(q[i] >> 16)), acc[2 * i + 1]);
      }
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (uint32_t)bf16_bits_rne(acc[2 * i]) | ((uint32_t)bf16_bits_rne(acc[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(out + t * ldo + n0) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_combine(const uint16_t* y, int64_t ldy, const int32_t* src_to_row, const float* w,
                          int64_t T, int32_t k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t st) {
  if (T == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, st, y, ldy, src_to_row, w, T, (int)k, N, out, ldo);
  return hipGetLastError();
}

}  // namespace fgg
