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
//   hist:    block b counts its kChunk pairs per expert (LDS atomics) into
//            hist[e][b]; the grid also sets row_to_src to -1.
//   scan:    one block per expert: exclusive prefix of hist[e][*] over blocks,
//            and the expert's total.
//   scatter: every block derives the padded segment offsets from the totals
//            (block 0 publishes them); block b then walks its pairs in order,
//            a pair's rank among equal experts coming from wave ballots
//            (stable) plus per-wave and per-block running counts.
//   gather:  one wave per row of [0, M_total) copies the token's codes (zeros
//            for padding rows); a second phase writes the K-block-major scales.
#include <mutex>

#include "fgg_device.hpp"
#include "fgg_internal.hpp"

namespace fgg {

static constexpr int kChunk = 256;    // pairs per block in hist/scatter (more, smaller blocks: measured faster than 512 or 1024)
static constexpr int kMaxE = 1024;

size_t permute_workspace_bytes(int64_t T, int32_t k, int32_t E) {
  const int64_t pairs = T * (int64_t)k;
  const int64_t nblk = (pairs + kChunk - 1) / kChunk;
  return (size_t)(nblk * (int64_t)E * sizeof(int32_t)) + 256;
}

__device__ inline int valid_expert(int e, int E) { return (e >= 0 && e < E) ? e : -1; }

// Inclusive sum over the 64 lanes of a wave.
__device__ inline int wave_inclusive_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__global__ void __launch_bounds__(256) permute_hist_kernel(const int32_t* __restrict__ ids, int64_t pairs,
                                                            int E, int64_t nblk, int32_t* __restrict__ hist,
                                                            int32_t* __restrict__ row_to_src, int64_t M_cap) {
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
  for (int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x; r < M_cap; r += (int64_t)gridDim.x * 256)
    row_to_src[r] = -1;
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(int64_t)e * nblk + blockIdx.x] = cnt[e];
}

__global__ void __launch_bounds__(256) fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// Block e: exclusive prefix of hist[e][0..nblk) in place; counts[e] = total.
__global__ void __launch_bounds__(256) permute_scan_kernel(int32_t* __restrict__ hist, int64_t nblk,
                                                            int32_t* __restrict__ counts) {
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* h = hist + (int64_t)blockIdx.x * nblk;
  int carry = 0;
  for (int64_t b0 = 0; b0 < nblk; b0 += 256) {
    const int64_t b = b0 + threadIdx.x;
    const int v = b < nblk ? h[b] : 0;
    const int incl = wave_inclusive_sum(v);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (b < nblk) h[b] = before + incl - v;
    carry += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) counts[blockIdx.x] = carry;
}

__global__ void __launch_bounds__(256) permute_scatter_kernel(const int32_t* __restrict__ ids, int64_t pairs,
                                                               int E, int align, int64_t nblk,
                                                               const int32_t* __restrict__ hist,
                                                               const int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ src_to_row,
                                                               int32_t* __restrict__ row_to_src, int64_t M_cap) {
  __shared__ int running[kMaxE];
  __shared__ int wave_cnt[4][kMaxE];
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Segment offsets: exclusive scan of the padded counts; thread t owns experts 4t..4t+3.
  {
    int pc[4], local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x * 4 + i;
      pc[i] = e < E ? ((counts[e] + align - 1) / align) * align : 0;
      local += pc[i];
    }
    const int incl = wave_inclusive_sum(local);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += wsum[w];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x * 4 + i;
      if (e < E) {
        running[e] = run + hist[(int64_t)e * nblk + blockIdx.x];
        if (blockIdx.x == 0) offsets[e] = run;
      }
      run += pc[i];
    }
    if (blockIdx.x == 0 && threadIdx.x == 255) offsets[E] = run;
  }
  for (int e = threadIdx.x; e < E; e += 256)
    wave_cnt[0][e] = wave_cnt[1][e] = wave_cnt[2][e] = wave_cnt[3][e] = 0;
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
      // a pair whose row falls at or beyond M_cap (M_cap too small) is reported as
      // dropped, so no consumer of src_to_row reads past the caller's buffers
      src_to_row[p] = before < M_cap ? before : -1;
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

// Rows [0, min(offsets[E], M_cap)): one wave per row copies the token's K code
// bytes (or zeros for a padding row), 8 x 16 B per lane in flight; then the
// K-block-major scales sa_out[kb][r] with consecutive threads on consecutive r.
__global__ void __launch_bounds__(256) permute_gather_kernel(const int32_t* __restrict__ offsets, int E, int k,
                                                              const int32_t* __restrict__ row_to_src,
                                                              const uint8_t* __restrict__ xq,
                                                              const float* __restrict__ xs, int64_t T,
                                                              int64_t K, uint8_t* __restrict__ a_out,
                                                              float* __restrict__ sa_out, int64_t M_cap) {
  int64_t m_total = offsets[E];
  if (m_total > M_cap) m_total = M_cap;
  const int lane = threadIdx.x & 63;
  const int64_t nvec = K / 16;
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t r = wave_id; r < m_total; r += nwaves) {
    const int32_t p = row_to_src[r];
    uint4* dst = reinterpret_cast<uint4*>(a_out + r * K);
    if (p >= 0) {
      const uint4* src = reinterpret_cast<const uint4*>(xq + (int64_t)(p / k) * K);
      for (int64_t i0 = lane; i0 < nvec; i0 += 64 * 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + 64 * u < nvec) v[u] = src[i0 + 64 * u];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + 64 * u < nvec) dst[i0 + 64 * u] = v[u];
      }
    } else {
      for (int64_t i = lane; i < nvec; i += 64) dst[i] = make_uint4(0, 0, 0, 0);
    }
  }
  const int64_t nkb = K / 128;
  const int64_t n = nkb * m_total;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t kb = i / m_total, r = i - kb * m_total;
    const int32_t p = row_to_src[r];
    sa_out[kb * M_cap + r] = p >= 0 ? xs[kb * T + p / k] : 0.0f;
  }
}

// Fused quantize + gather: the same outputs as quantizing x to e4m3 with 1x128
// scales and then gathering the codes (the permute_gather_kernel contract),
// without writing or re-reading the token-order codes.  One wave per (token,
// column batch): lane j < k holds slot j's destination row; a token with no
// destination below M_cap is not read at all.  The batch is kPermPB passes of
// 1024 columns (8 lanes x 16 elements per 128-column group), all loaded before
// the first is used; each pass's codes (16 bytes per lane) and scales go to
// every destination row.  A second phase zero-fills the padding rows of [0, M_total).
// Raw bytes of 8 consecutive elements: one 16-byte load for bf16, two for fp32.
template <bool BF16>
struct RawRow8;
template <>
struct RawRow8<true> {
  uint4 a;
};
template <>
struct RawRow8<false> {
  uint4 a, b;
};

template <bool BF16>
__device__ inline RawRow8<BF16> load_raw8(const void* base, int64_t idx) {
  RawRow8<BF16> r;
  if constexpr (BF16) {
    r.a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
  } else {
    const uint4* q = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + idx);
    r.a = q[0];
    r.b = q[1];
  }
  return r;
}

template <bool BF16>
__device__ inline void unpack_raw8(const RawRow8<BF16>& r, float* f) {
  if constexpr (BF16) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
      f[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  } else {
    f[0] = __uint_as_float(r.a.x); f[1] = __uint_as_float(r.a.y);
    f[2] = __uint_as_float(r.a.z); f[3] = __uint_as_float(r.a.w);
    f[4] = __uint_as_float(r.b.x); f[5] = __uint_as_float(r.b.y);
    f[6] = __uint_as_float(r.b.z); f[7] = __uint_as_float(r.b.w);
  }
}

// Columns of one token quantized by one wave: kPermPB passes of 1024 (each lane 16
// columns per pass), all loaded before the first conversion.  One such item per wave and
// no loop over items: a wave that looped would wait, at its next item's loads, for its
// previous stores as well (with loads and stores both outstanding the vector-memory
// counter gives no order, so the wait is for all of them), while a retiring wave's
// stores drain on their own and its slot takes the next item.
constexpr int kPermPB = 1;

template <bool BF16>
__global__ void __launch_bounds__(256) permute_quantize_kernel(const int32_t* __restrict__ offsets, int E, int k,
                                                                const int32_t* __restrict__ src_to_row,
                                                                const int32_t* __restrict__ row_to_src,
                                                                const void* __restrict__ x, int64_t ldx,
                                                                int64_t T, int64_t K,
                                                                uint8_t* __restrict__ a_out,
                                                                float* __restrict__ sa_out, int64_t M_cap) {
  const int lane = threadIdx.x & 63, sub = lane & 7;
  const int64_t wave_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int64_t nbat = (K + 1024 * kPermPB - 1) / (1024 * kPermPB);
  // one work item per wave: token t, columns [c0, c0 + 1024 kPermPB)
  if (wave_id < T * nbat) {
    const int64_t t = wave_id / nbat, c0 = (wave_id - t * nbat) * (1024 * kPermPB);
    const int32_t dst = lane < k ? src_to_row[t * k + lane] : -1;
    const uint64_t dmask = __ballot(dst >= 0 && dst < M_cap);
    if (dmask != 0) {
      constexpr int kPB = kPermPB;
      RawRow8<BF16> raw[kPB][2];
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        const int64_t col = c0 + 1024 * pb + 16 * lane;
        if (col < K) {
          raw[pb][0] = load_raw8<BF16>(x, t * ldx + col);
          raw[pb][1] = load_raw8<BF16>(x, t * ldx + col + 8);
        }
      }
#pragma unroll
      for (int pb = 0; pb < kPB; ++pb) {
        const int64_t col = c0 + 1024 * pb + 16 * lane;
        if (c0 + 1024 * pb >= K) break;             // wave-uniform
        const bool live = col < K;                  // uniform per 8-lane group (K % 128 == 0)
        float v[16];
        if (live) {
          unpack_raw8<BF16>(raw[pb][0], v);
          unpack_raw8<BF16>(raw[pb][1], v + 8);
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) v[i] = 0.0f;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
        amax = group_max<8>(amax);
        const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
        const float r = __builtin_amdgcn_rcpf(s);
        float y[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = e4m3_quotient(v[i], s, r);
        const uint4 codes = make_uint4(e4m3_pack4(y[0], y[1], y[2], y[3]), e4m3_pack4(y[4], y[5], y[6], y[7]),
                                       e4m3_pack4(y[8], y[9], y[10], y[11]), e4m3_pack4(y[12], y[13], y[14], y[15]));
        const int64_t kb = col >> 7;
        uint64_t m = dmask;
        while (m) {
          const int j = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const int64_t row = __shfl(dst, j);
          if (live) {
            *reinterpret_cast<uint4*>(a_out + row * K + col) = codes;
            if (sub == 0) sa_out[kb * M_cap + row] = s;
          }
        }
      }
    }
  }
  int64_t m_total = offsets[E];
  if (m_total > M_cap) m_total = M_cap;
  const int64_t nvec = K / 16, nkb = K / 128;
  for (int64_t r = wave_id; r < m_total; r += nwaves) {
    if (row_to_src[r] >= 0) continue;   // wave-uniform
    uint4* d = reinterpret_cast<uint4*>(a_out + r * K);
    for (int64_t i = lane; i < nvec; i += 64) d[i] = make_uint4(0, 0, 0, 0);
    for (int64_t kb = lane; kb < nkb; kb += 64) sa_out[kb * M_cap + r] = 0.0f;
  }
}

const KernelInfo kInfoPermuteHist = {"permute_hist_kernel", "fgg_moe_permute, fgg_moe_permute_quantize", 0, 0, 0,
                                     256, 0, 0, kMaxE * 4, kMaxE * 4, (const void*)permute_hist_kernel};
const KernelInfo kInfoPermuteScan = {"permute_scan_kernel", "fgg_moe_permute, fgg_moe_permute_quantize", 0, 0, 0,
                                     256, 0, 0, 16, 16, (const void*)permute_scan_kernel};
const KernelInfo kInfoPermuteScatter = {"permute_scatter_kernel", "fgg_moe_permute, fgg_moe_permute_quantize", 0, 0,
                                        0, 256, 0, 0, kMaxE * 4 * 5 + 16, kMaxE * 4 * 5 + 16,
                                        (const void*)permute_scatter_kernel};
const KernelInfo kInfoPermuteGather = {"permute_gather_kernel", "fgg_moe_permute", 0, 0, 0, 256, 0, 0, 0, 0,
                                       (const void*)permute_gather_kernel};
const KernelInfo kInfoPermuteQuantize = {"permute_quantize_kernel", "fgg_moe_permute_quantize", 1, 128, 128, 256, 0,
                                         0, 0, 0, (const void*)permute_quantize_kernel<true>};
const KernelInfo kInfoFill = {"fill_i32_kernel", "fgg_moe_permute (T == 0)", 0, 0, 0, 256, 0, 0, 0, 0,
                              (const void*)fill_i32_kernel};

hipError_t launch_permute(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t align,
                          const uint8_t* xq, const float* xs, int64_t K, int32_t* offsets,
                          int32_t* counts, int32_t* src_to_row, int32_t* row_to_src, uint8_t* a_out,
                          float* sa_out, int64_t M_cap, void* ws, hipStream_t st) {
  const int64_t pairs = T * (int64_t)k;
  if (pairs == 0) {
    trace_launch(kInfoFill, dim3(1), "T=0 E=%d M_cap=%lld", (int)E, (long long)M_cap);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, offsets, (int64_t)E + 1, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, counts, (int64_t)E, 0);
    if (M_cap > 0)
      hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((M_cap + 255) / 256 < 1024 ? (M_cap + 255) / 256 : 1024)), dim3(256), 0, st, row_to_src, M_cap, -1);
    return hipGetLastError();
  }
  const int64_t nblk = (pairs + kChunk - 1) / kChunk;
  int32_t* hist = reinterpret_cast<int32_t*>(ws);
  trace_launch(kInfoPermuteHist, dim3((unsigned)nblk), "pairs=%lld E=%d M_cap=%lld", (long long)pairs, (int)E,
               (long long)M_cap);
  trace_launch(kInfoPermuteScan, dim3((unsigned)E), "blocks=%lld", (long long)nblk);
  trace_launch(kInfoPermuteScatter, dim3((unsigned)nblk), "pairs=%lld align=%d", (long long)pairs, (int)align);
  hipLaunchKernelGGL(permute_hist_kernel, dim3((unsigned)nblk), dim3(256), 0, st, ids, pairs, (int)E, nblk, hist,
                     row_to_src, M_cap);
  hipLaunchKernelGGL(permute_scan_kernel, dim3((unsigned)E), dim3(256), 0, st, hist, nblk, counts);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)nblk), dim3(256), 0, st, ids, pairs, (int)E,
                     (int)align, nblk, hist, counts, offsets, src_to_row, row_to_src, M_cap);
  if (xq != nullptr && M_cap > 0) {
    trace_launch(kInfoPermuteGather, dim3(1024), "K=%lld M_cap=%lld", (long long)K, (long long)M_cap);
    hipLaunchKernelGGL(permute_gather_kernel, dim3(1024), dim3(256), 0, st, offsets, (int)E, (int)k, row_to_src,
                       xq, xs, T, K, a_out, sa_out, M_cap);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate (fgg_moe_permute_quantize_noalloc):
// the per-block expert histograms live in this file-scope device array instead of
// a caller workspace.  Each device that runs the library holds its own copy for
// the life of the process; its address is taken per device with
// hipGetSymbolAddress (the array's name is only a host-side stand-in).  Every
// histogram entry is written before it is read, so nothing is cleared between
// calls; calls that overlap on one device share the array and race.
static __device__ __align__(256) uint8_t scratch[kPermuteScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];
}  // namespace

hipError_t permute_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (g_scratch_ptr[dev] == nullptr) return hipErrorInvalidSymbol;
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_permute_quantize(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t align,
                                   const void* x, bool bf16, int64_t K, int64_t ldx, int32_t* offsets,
                                   int32_t* counts, int32_t* src_to_row, int32_t* row_to_src, uint8_t* a_out,
                                   float* sa_out, int64_t M_cap, void* ws, int num_cus, hipStream_t st) {
  hipError_t e = launch_permute(ids, T, k, E, align, nullptr, nullptr, K, offsets, counts, src_to_row,
                                row_to_src, nullptr, nullptr, M_cap, ws, st);
  if (e != hipSuccess || T == 0 || M_cap == 0) return e;
  (void)num_cus;
  const int64_t nbat = (K + 1024 * kPermPB - 1) / (1024 * kPermPB);
  const int64_t blocks = (T * nbat + 3) / 4;                // one (token, column batch) item per wave
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const unsigned grid = (unsigned)blocks;
  trace_launch(kInfoPermuteQuantize, dim3(grid), "T=%lld K=%lld %s M_cap=%lld", (long long)T, (long long)K,
               bf16 ? "bf16" : "fp32", (long long)M_cap);
  if (bf16)
    hipLaunchKernelGGL(permute_quantize_kernel<true>, dim3(grid), dim3(256), 0, st, offsets, (int)E, (int)k,
                       src_to_row, row_to_src, x, ldx, T, K, a_out, sa_out, M_cap);
  else
    hipLaunchKernelGGL(permute_quantize_kernel<false>, dim3(grid), dim3(256), 0, st, offsets, (int)E, (int)k,
                       src_to_row, row_to_src, x, ldx, T, K, a_out, sa_out, M_cap);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: one 256-thread block per token.  A thread owns 16-byte column
// chunks n = 8 * (256 c + tid), four chunks per pass; for each routed slot in
// increasing j it loads all of its chunks of that row at once, then
// accumulates them with fp32 FMA (the same order for every column).
// Routing table of the down GEMM's combine epilogue: per permuted row r < M, the token
// of its slot and the slot's gate weight when that token has exactly one routed slot
// (then the row is the token's whole output), else token -1 (padding rows, rows past the
// routed ones, and rows of tokens with two or more routed slots).
__global__ void __launch_bounds__(256) combine_rows_kernel(const int32_t* __restrict__ row_to_src,
                                                            const int32_t* __restrict__ src_to_row,
                                                            const float* __restrict__ w, int64_t T, int k,
                                                            int64_t M, uint2* __restrict__ row_info) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= M) return;
  const int32_t p = row_to_src[r];
  uint2 e = make_uint2(0xFFFFFFFFu, 0u);
  if (p >= 0 && (int64_t)p < T * k) {
    const int64_t t = p / k;
    int routed = 0;
    for (int j = 0; j < k; ++j) routed += src_to_row[t * k + j] >= 0;
    if (routed == 1) e = make_uint2((uint32_t)t, __float_as_uint(w[p]));
  }
  row_info[r] = e;
}

// SKIP_SINGLE: tokens with exactly one routed slot are left alone (the down GEMM's
// combine epilogue wrote their output rows).
template <bool SKIP_SINGLE>
__global__ void __launch_bounds__(256) combine_kernel(const uint16_t* __restrict__ y, int64_t ldy,
                                                       const int32_t* __restrict__ src_to_row,
                                                       const float* __restrict__ w, int64_t T, int k,
                                                       int64_t N, uint16_t* __restrict__ out, int64_t ldo) {
  constexpr int C = 4;
  const int64_t t = blockIdx.x;
  if constexpr (SKIP_SINGLE) {
    int routed = 0;
    for (int j = 0; j < k; ++j) routed += src_to_row[t * k + j] >= 0;
    if (routed == 1) return;
  }
  for (int64_t base = 0; base < N; base += C * 2048) {
    float acc[C][8];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[c][i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int32_t row = src_to_row[t * k + j];
      if (row < 0) continue;
      const float wj = w[t * k + j];
      const uint16_t* yr = y + (int64_t)row * ldy;
      uint4 u[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int64_t n0 = base + 8 * (256 * c + threadIdx.x);
        if (n0 < N) u[c] = *reinterpret_cast<const uint4*>(yr + n0);
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const uint32_t q[4] = {u[c].x, u[c].y, u[c].z, u[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[c][2 * i] = fmaf(wj, bf16_to_f32((uint16_t)(q[i] & 0xFFFFu)), acc[c][2 * i]);
          acc[c][2 * i + 1] = fmaf(wj, bf16_to_f32((uint16_t)(q[i] >> 16)), acc[c][2 * i + 1]);
        }
      }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int64_t n0 = base + 8 * (256 * c + threadIdx.x);
      if (n0 < N) {
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = bf16x2_rne(acc[c][2 * i], acc[c][2 * i + 1]);
        *reinterpret_cast<uint4*>(out + t * ldo + n0) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

const KernelInfo kInfoCombine = {"combine_kernel", "fgg_moe_combine", 0, 0, 0, 256, 0, 0, 0, 0,
                                 (const void*)combine_kernel<false>};
const KernelInfo kInfoCombineRest = {"combine_kernel<skip single>", "fgg_moe_down_combine", 0, 0, 0, 256, 0, 0, 0,
                                     0, (const void*)combine_kernel<true>};
const KernelInfo kInfoCombineRows = {"combine_rows_kernel", "fgg_moe_down_combine", 0, 0, 0, 256, 0, 0, 0, 0,
                                     (const void*)combine_rows_kernel};

hipError_t launch_combine(const uint16_t* y, int64_t ldy, const int32_t* src_to_row, const float* w,
                          int64_t T, int32_t k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t st) {
  if (T == 0 || N == 0) return hipSuccess;
  trace_launch(kInfoCombine, dim3((unsigned)T), "T=%lld k=%d N=%lld", (long long)T, (int)k, (long long)N);
  hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)T), dim3(256), 0, st, y, ldy, src_to_row, w, T, (int)k, N,
                     out, ldo);
  return hipGetLastError();
}

hipError_t launch_combine_rows(const int32_t* row_to_src, const int32_t* src_to_row, const float* w, int64_t T,
                               int32_t k, int64_t M, uint8_t* row_info, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const int64_t blocks = (M + 255) / 256;
  trace_launch(kInfoCombineRows, dim3((unsigned)blocks), "M=%lld T=%lld k=%d", (long long)M, (long long)T, (int)k);
  hipLaunchKernelGGL(combine_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, row_to_src, src_to_row, w, T,
                     (int)k, M, reinterpret_cast<uint2*>(row_info));
  return hipGetLastError();
}

hipError_t launch_combine_rest(const uint16_t* y, int64_t ldy, const int32_t* src_to_row, const float* w, int64_t T,
                               int32_t k, int64_t N, uint16_t* out, int64_t ldo, hipStream_t st) {
  if (T == 0 || N == 0) return hipSuccess;
  trace_launch(kInfoCombineRest, dim3((unsigned)T), "T=%lld k=%d N=%lld", (long long)T, (int)k, (long long)N);
  hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)T), dim3(256), 0, st, y, ldy, src_to_row, w, T, (int)k, N,
                     out, ldo);
  return hipGetLastError();
}

}  // namespace fgg
